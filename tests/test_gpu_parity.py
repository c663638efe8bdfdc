"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Attention: max |out - oracle| <= 2e-3 and max |lse - oracle| <= 1e-4 over
live rows, at the page's fp32-faithful probabilities (probability_parts = 3,
the default) and also with 2 parts; padding rows exactly 0 / -inf; no NaN
although every dead cache slot, padding query, logits row and draft row holds
NaN. The lossy fast mode (probability_parts = 1) is tested only by the tests
whose names say "fast_mode", against the bound include/tv.h states for it. Mask and greedy
outputs: bit-exact. Sampling: bit-exact decisions except within 1e-6 of a
threshold.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.decode import decode
from workloads import make_config, make_custom
from workloads.gen import bf16_bits_from_f32

from gpu_util import (ATOL_OUT, check_attention, check_greedy, check_sample, fast_mode_bound,
                      oracle_attention, run_attention, run_greedy, run_mask, run_sample, upload)
import tree_attention_draft_tv_amd as tv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    tv.load()


def _mask_check(w, d):
    mask, depth, st = run_mask(d, w.T)
    torch.cuda.synchronize()
    m_ref, dep_ref, st_ref = oracle.build_tree_mask(w.parent, w.n_nodes, w.T)
    assert np.array_equal(st.cpu().numpy(), st_ref)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), m_ref)
    assert np.array_equal(depth.cpu().numpy(), dep_ref)
    return mask


# ------------------------------------------------------------------ mask ---

@pytest.mark.parametrize("T", [1, 2, 9, 33, 64, 65, 100, 128])
def test_mask_random_trees(T):
    rng = np.random.default_rng(T)
    B = 6
    parent = np.full((B, T), -1, np.int32)
    n_nodes = np.array([T, T, max(T - 3, 0), 0, T, T], np.int32)
    for b in range(B):
        for i in range(1, T):
            if b == 4:
                parent[b, i] = i - 1                # chain
            elif b == 5:
                parent[b, i] = 0                    # star
            else:
                parent[b, i] = rng.integers(0, i)
    d = {"parent": torch.from_numpy(parent).cuda(), "n_nodes": torch.from_numpy(n_nodes).cuda()}

    class W:
        pass
    w = W()
    w.parent, w.n_nodes, w.T = parent, n_nodes, T
    _mask_check(w, d)


def test_mask_status_codes():
    T = 8
    parent = np.tile(np.arange(-1, T - 1, dtype=np.int32), (4, 1))
    parent[1, 5] = 5          # not < 5
    parent[2, 3] = -2
    n_nodes = np.array([8, 8, 8, 9], np.int32)
    d = {"parent": torch.from_numpy(parent).cuda(), "n_nodes": torch.from_numpy(n_nodes).cuda()}

    class W:
        pass
    w = W()
    w.parent, w.n_nodes, w.T = parent, n_nodes, T
    _mask_check(w, d)


# ------------------------------------------------------------- attention ---

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_attention_configs(name):
    # Every workload at the page's precision: fp32-faithful probabilities
    # (three bf16 parts) and fp32 split partials.
    w = make_config(name)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, parts=3)
    check_attention(w, got, oracle_attention(w), label=name)


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_attention_fast_mode_configs(name):
    # The lossy fast mode on the measured workloads, against its stated bound.
    w = make_config(name)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, parts=1)
    check_attention(w, got, oracle_attention(w), atol_out=fast_mode_bound(w),
                    label=name + " fast mode")


def _ragged_case(dtype, D, chunk):
    # Ragged contexts (not multiples of the chunk or the 64-key tile), an empty
    # context (only tree keys visible), a partial tree, a padded sequence, a
    # root-only tree, G = 3 so packed rows straddle MFMA tiles.
    return make_custom(31 + D + chunk, 5, 9, 3, D, 50, dtype, [300, 0, 77, 1000, 129], 20,
                       n_nodes=[21, 21, 13, 0, 1], trie_tokens=False)


@pytest.mark.parametrize("dtype,parts", [("bf16", 3), ("bf16", 2), ("f32", 3)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("chunk", [64, 128, 0])
def test_attention_multichunk_ragged(dtype, parts, D, chunk):
    w = _ragged_case(dtype, D, chunk)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
    err_o, _ = check_attention(w, got, oracle_attention(w), label="%s parts=%d" % (dtype, parts))
    assert err_o < 5e-5, err_o  # fp32 (or 16-bit) probabilities: accumulation error only


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("chunk", [64, 0])
def test_attention_fast_mode_multichunk_ragged(D, chunk):
    w = _ragged_case("bf16", D, chunk)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=chunk, parts=1)
    check_attention(w, got, oracle_attention(w), atol_out=fast_mode_bound(w), label="fast mode")


@pytest.mark.parametrize("parts", [2, 3])
def test_attention_probability_parts(parts):
    w = make_custom(41, 2, 16, 2, 128, 50, "bf16", [37, 700], 40, max_depth=10,
                    trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=256, parts=parts)
    err_o, err_l = check_attention(w, got, oracle_attention(w), label="parts=%d" % parts)
    if parts == 3:  # probabilities fp32-faithful: only fp32 accumulation error remains
        assert err_o < 2e-5 and err_l < 2e-5, (err_o, err_l)


def test_attention_fast_mode_probability_parts():
    w = make_custom(41, 2, 16, 2, 128, 50, "bf16", [37, 700], 40, max_depth=10,
                    trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=256, parts=1)
    check_attention(w, got, oracle_attention(w), atol_out=fast_mode_bound(w), label="fast mode")


def _runaway_case(where):
    # One key is 8x a query vector, so its score lies far above those of the
    # first keys of its unit: probabilities against that first-keys reference
    # would run past 2^32, and the unit is redone against its exact max.
    w = make_custom(111, 2, 14, 2, 128, 50, "bf16", [1500, 90], 32, trie_tokens=False)
    qf = decode(w.q, w.dtype)
    b, node, h = 0, 5, 3
    key = 700 if where == "committed" else int(w.ctx_len[b]) + node
    w.k[b, h // w.G, key] = bf16_bits_from_f32(8.0 * qf[b, node, h])
    want = oracle_attention(w)
    row = want[0][b, node, h]
    assert np.abs(row - decode(w.v, w.dtype)[b, h // w.G, key]).max() < 1e-3  # one key dominates
    return w, want


@pytest.mark.parametrize("where,parts", [("committed", 3), ("committed", 2), ("tree", 3),
                                         ("tree", 2)])
def test_attention_runaway_scores_redone_with_exact_max(where, parts):
    # One key is 8x a query vector, so its score lies far above those of the
    # first keys of its unit: probabilities against that first-keys reference
    # would run past 2^32, and the unit is redone against its exact max.
    w, want = _runaway_case(where)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=512, parts=parts)
    check_attention(w, got, want, label="%s parts=%d" % (where, parts))


@pytest.mark.parametrize("where", ["committed", "tree"])
def test_attention_fast_mode_runaway_scores(where):
    w, want = _runaway_case(where)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=512, parts=1)
    check_attention(w, got, want, atol_out=fast_mode_bound(w), label="%s fast mode" % where)


@pytest.mark.parametrize("chunk", [256, 0])
def test_attention_fast_mode_fixed_point_partials_error_bound(chunk):
    # Every (node, head) row attends to one committed key of its own: its
    # query is a multiple of that key, so the key's score lies ~28 above all
    # others and its one-part probability is exactly 1 (the rest ~1e-12).
    # Values are large (|v| up to ~300), so what is left of the error is the
    # 16-bit fixed point of the split partials: at most max|v| / 65534 per
    # entry. With two parts the partials stay fp32 and the error is tiny.
    w = make_custom(131, 1, 7, 1, 128, 50, "bf16", [2000], 8, trie_tokens=False)
    rng = np.random.default_rng(17)
    kf = decode(w.k, w.dtype)
    vf = decode(w.v, w.dtype)
    qf = decode(w.q, w.dtype)
    n, L = int(w.n_nodes[0]), int(w.ctx_len[0])
    live = L + n
    w.v[0, 0, :live] = bf16_bits_from_f32(64.0 * vf[0, 0, :live])
    target = rng.integers(0, L, size=(n, w.Hq))
    for i in range(n):
        for h in range(w.Hq):
            kk = kf[0, 0, target[i, h]]
            alpha = 40.0 / (float(w.scale) * float(kk @ kk))
            qf[0, i, h] = alpha * kk
    w.q[0, :n] = bf16_bits_from_f32(qf[0, :n])
    d = upload(w)
    mask = _mask_check(w, d)
    want = oracle_attention(w)
    vmax = np.abs(decode(w.v, w.dtype)[0, 0, :live]).max()
    bound = vmax / 65534.0
    got1 = run_attention(w, d, mask, chunk_keys=chunk, parts=1)
    err1 = np.abs(got1[0][0, :n] - want[0][0, :n]).max()
    assert err1 <= bound * 1.001 + 1e-4, (err1, bound)
    assert np.abs(got1[1][0, :n] - want[1][0, :n]).max() <= 1e-4
    for parts in (2, 3):  # fp32 partials: the page's precision holds 2e-3 at |v| ~ 300
        got2 = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
        err2 = np.abs(got2[0][0, :n] - want[0][0, :n]).max()
        assert err2 <= 2e-4, (parts, err2)
        check_attention(w, got2, want, label="|v| ~ 300, parts=%d" % parts)


def test_attention_many_rows_two_row_groups():
    # R = 16 heads per KV head x 65 rows = 1040 packed rows: five row groups.
    w = make_custom(51, 1, 16, 1, 128, 50, "bf16", [333], 64, max_depth=12, max_children=6,
                    trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    want = oracle_attention(w)
    for chunk in (64, 0):
        got = run_attention(w, d, mask, chunk_keys=chunk)
        check_attention(w, got, want, label="chunk %d" % chunk)


def test_attention_context_bound_status():
    w = make_custom(61, 3, 4, 2, 64, 50, "bf16", [100, 200, 50], 8, trie_tokens=False,
                    max_ctx=150, kv_capacity=256)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=64)
    want = oracle.tree_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, w.parent,
                                 w.scale, max_ctx=150, kv_capacity=256)
    assert want[2].tolist() == [0, oracle.ROW_CTX_BOUND, 0]
    check_attention(w, got, want)


def test_attention_batch_invariance_and_determinism():
    w = make_custom(71, 4, 14, 2, 128, 50, "bf16", [900, 2000, 64, 1500], 32,
                    trie_tokens=False, n_nodes=[33, 33, 20, 33])
    d = upload(w)
    mask = _mask_check(w, d)
    a = run_attention(w, d, mask, chunk_keys=256, max_ctx=2048)
    b2 = run_attention(w, d, mask, chunk_keys=256, max_ctx=2048)
    assert np.array_equal(a[0], b2[0]) and np.array_equal(a[1], b2[1])
    for b in range(w.B):
        sl = slice(b, b + 1)
        one = {k: (v[sl] if v.dim() > 0 else v) for k, v in d.items()}
        m1 = mask[sl].contiguous()
        o1, l1, _ = tv.tree_attention(one["q"], one["k"], one["v"], one["ctx_len"],
                                      one["n_nodes"], m1, 2048, scale=float(w.scale),
                                      chunk_keys=256)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0], a[0][b])
        assert np.array_equal(l1.cpu().numpy()[0], a[1][b])


@pytest.mark.parametrize("name,chunk", [("C2", 0), ("C3", 512), ("C3", 768)])
def test_attention_repeated_calls_bitwise_identical(name, chunk):
    # C2's last chunks hold the tree block across two masked tiles after a
    # pipelined one: every tile must have landed in LDS before it is read,
    # whatever the timing of the copies, so repeated calls agree bit for bit.
    w = make_config(name)
    d = upload(w)
    mask = _mask_check(w, d)
    first = run_attention(w, d, mask, chunk_keys=chunk)
    for _ in range(10):
        again = run_attention(w, d, mask, chunk_keys=chunk)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_attention_chunk_size_invariance_fp32_faithful():
    w = make_custom(81, 2, 7, 1, 128, 50, "bf16", [1000, 3000], 32, trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    ref = run_attention(w, d, mask, chunk_keys=64, parts=3)
    for chunk in (128, 512, 4096):
        got = run_attention(w, d, mask, chunk_keys=chunk, parts=3)
        assert np.abs(got[0] - ref[0]).max() < 1e-5
        assert np.abs(got[1] - ref[1]).max() < 1e-5


def test_attention_strided_nhd_cache():
    # Cache laid out [B][capacity][Hkv][D] (NHD) and viewed through strides.
    w = make_custom(91, 2, 8, 2, 128, 50, "bf16", [200, 90], 12, trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    k_nhd = d["k"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v_nhd = d["v"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out, lse, st = tv.tree_attention(d["q"], k_nhd, v_nhd, d["ctx_len"], d["n_nodes"], mask,
                                     w.max_ctx, scale=float(w.scale), chunk_keys=64)
    torch.cuda.synchronize()
    check_attention(w, (out.cpu().numpy(), lse.cpu().numpy(), st.cpu().numpy()),
                    oracle_attention(w), label="NHD")


def test_attention_all_padded_batch():
    w = make_custom(95, 3, 4, 1, 64, 50, "bf16", [10, 20, 30], 5, trie_tokens=False,
                    padded_rows=[0, 1, 2])
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=64)
    check_attention(w, got, oracle_attention(w))


# ---------------------------------------------------------------- greedy ---

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_greedy_configs(name):
    w = make_config(name)
    d = upload(w)
    got = run_greedy(d)
    want = oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes)
    check_greedy(got, want)
    for b in w.planted:
        assert got[0][b] == 4 and list(got[1][b, :5]) == w.planted[b]


@pytest.mark.parametrize("V", [1, 3, 4, 5, 1000, 16387, 40000])
def test_greedy_ties_and_odd_vocab(V):
    rng = np.random.default_rng(V)
    w = make_custom(V, 4, 2, 1, 64, V, "bf16", [4, 4, 4, 4], 12, trie_tokens=False,
                    padded_rows=[2])
    logits = w.logits.copy()
    for b in range(4):
        for j in range(int(w.n_nodes[b])):
            row = logits[b, j]
            m = row.max()
            # plant exact ties of the maximum at several positions, and signed zeros
            k = rng.integers(1, 4)
            pos = rng.choice(V, size=min(k, V), replace=False)
            row[pos] = m + 1.0
            if j % 3 == 0:
                row[:] = np.where(rng.random(V) < 0.5, np.float32(-0.0), np.float32(0.0))
                row[rng.integers(0, V, size=max(1, V // 4))] = -1.0
    # make some draft tokens match so the walk goes deeper
    for b in range(4):
        for c in range(1, int(w.n_nodes[b])):
            if rng.random() < 0.6:
                row = logits[b, w.parent[b, c]].astype(np.float64)
                w.tokens[b, c] = int(np.flatnonzero(row == row.max())[0])
    w.logits = logits
    d = upload(w)
    got = run_greedy(d)
    check_greedy(got, oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes))


def test_greedy_status_codes():
    w = make_custom(5, 4, 2, 1, 64, 100, "bf16", [4] * 4, 6, trie_tokens=False)
    w.parent[1, 3] = 4
    w.tokens[2, 2] = 100
    w.n_nodes[3] = 9
    d = upload(w)
    got = run_greedy(d)
    want = oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes)
    assert want[4].tolist() == [0, oracle.ROW_BAD_PARENT, oracle.ROW_BAD_TOKEN, oracle.ROW_NNODES]
    check_greedy(got, want)


def _greedy_shapes(seed):
    # Same launch shape for every seed; the planted argmax paths differ.
    return make_custom(seed, 6, 2, 1, 64, 40000, "bf16", [4] * 6, 24, plant_depth=4,
                       padded_rows=[2])


def test_greedy_workspace_reuse():
    # One workspace of random bytes for calls of two launch shapes in turn:
    # every call's partials are its own.
    ws = torch.randint(0, 256, (1 << 22,), dtype=torch.uint8, device=torch.device("cuda:0"))
    a, b = _greedy_shapes(41), _greedy_shapes(42)
    other = make_custom(43, 3, 2, 1, 64, 100000, "bf16", [4] * 3, 40, plant_depth=3)
    for w in (a, b, other, a, b, a):
        d = upload(w)
        res = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"], workspace=ws)
        torch.cuda.synchronize()
        got = tuple(r.cpu().numpy() for r in res)
        check_greedy(got, oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes))


def test_greedy_graph_replays_with_new_logits():
    # Replays of one captured call, with new inputs copied in before each.
    ws = [_greedy_shapes(50 + r) for r in range(4)]
    d = upload(ws[0])
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g):
            acc = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(8):
        w = ws[rep % 4]
        e = upload(w)
        for key in ("logits", "tokens", "parent", "n_nodes"):
            d[key].copy_(e[key])
        acc[0].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = tuple(x.cpu().numpy() for x in acc)
        check_greedy(got, oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes))


# -------------------------------------------------------------- sampling ---

def test_sample_config_c5():
    w = make_config("C5")
    d = upload(w)
    got = run_sample(w, d)
    want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                w.n_nodes)
    exempt = check_sample(w, got, want)
    print("C5 sampling: exempt rows", exempt)
    assert exempt <= 1


@pytest.mark.parametrize("seed", range(4))
def test_sample_small_vocab_many_rows(seed):
    w = make_custom(200 + seed, 16, 2, 1, 64, 7, "bf16", [4] * 16, 10, mode="sample",
                    temperature=0.9 + 0.3 * seed, padded_rows=[3])
    # make some draft probabilities exactly zero and some rows one-hot
    rng = np.random.default_rng(seed)
    for b in range(16):
        for c in range(1, 11):
            if rng.random() < 0.3:
                z = rng.integers(0, 7)
                if z != w.tokens[b, c]:
                    w.qdraft[b, c, z] = 0.0
            if rng.random() < 0.15:
                w.qdraft[b, c] = 0.0
                w.qdraft[b, c, w.tokens[b, c]] = 1.0
    d = upload(w)
    got = run_sample(w, d)
    want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                w.n_nodes)
    assert check_sample(w, got, want) <= 1


@pytest.mark.parametrize("V", [1, 1000, 3000, 32768, 32769, 40000])
def test_sample_vocab_sizes(V):
    """Vocabularies on both sides of the one-round-trip walk's limit (32768
    entries), with ragged tails: star trees force several rejections at the
    root (residual chains), random trees mix acceptances in."""
    for seed, tree in ((300, "star"), (301, "random")):
        w = make_custom(seed + V, 3, 2, 1, 64, V, "bf16", [8] * 3, 12, mode="sample",
                        tree=tree, temperature=0.8)
        d = upload(w)
        got = run_sample(w, d)
        want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                    w.n_nodes)
        assert check_sample(w, got, want) <= 1


@pytest.mark.parametrize("seed", range(11000, 11024))
def test_sample_random_cases(seed):
    # Seeded draws: batch, tree size and shape, vocabularies on both sides of
    # the one-round-trip limit, temperature, padded sequences, and draft rows
    # with zeroed entries or all their mass on the drafted token.
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 13))
    nd = int(rng.integers(0, 60))
    V = int(rng.choice([int(rng.integers(1, 50)), int(rng.integers(50, 33000)),
                        int(rng.integers(32700, 70000))]))
    tau = float(rng.uniform(0.3, 2.0))
    tree = str(rng.choice(["random", "random", "star", "chain"]))
    padded = [b for b in range(B) if rng.random() < 0.15]
    w = make_custom(seed, B, 2, 1, 64, V, "bf16", [4] * B, nd, mode="sample", tree=tree,
                    temperature=tau, padded_rows=padded)
    for b in range(B):
        for c in range(1, nd + 1):
            r = rng.random()
            if r < 0.1:
                z = int(rng.integers(0, V))
                if z != w.tokens[b, c]:
                    w.qdraft[b, c, z] = 0.0
            elif r < 0.15:
                w.qdraft[b, c] = 0.0
                w.qdraft[b, c, w.tokens[b, c]] = 1.0
    d = upload(w)
    got = run_sample(w, d)
    want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                w.n_nodes)
    assert check_sample(w, got, want) <= 1


def test_sample_unnormalised_draft_keeps_residual():
    """A draft row that dominates the residual everywhere (q = 2 r) leaves a
    zero residual sum, so r is kept; later siblings are tested against it."""
    V = 500
    w = make_custom(77, 2, 2, 1, 64, V, "bf16", [8] * 2, 4, mode="sample", tree="star",
                    temperature=1.0)
    p0 = [oracle.sample_probs(w.logits[b, 0], w.temperature) for b in range(2)]
    for b in range(2):
        w.qdraft[b, 1] = (2.0 * p0[b]).astype(np.float32)
        w.u[b, 1] = 0.75  # ratio = 1/2 -> rejected
    d = upload(w)
    got = run_sample(w, d)
    want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                w.n_nodes)
    assert np.all(want[4][:, 1] == 0)
    assert check_sample(w, got, want) == 0


def test_sample_draws_follow_target():
    """Statistical check of the GPU sampler itself: the first emitted token
    over many independent rows follows p_root (chi-square)."""
    import scipy.stats
    rng = np.random.default_rng(9)
    V, rows, k = 5, 4096, 3
    T = k + 1
    root = np.log(rng.dirichlet(np.ones(V))).astype(np.float32)
    logits = np.tile(root, (rows, T, 1)).astype(np.float32)
    q = np.full((rows, T, V), np.nan, np.float32)
    tokens = np.zeros((rows, T), np.int32)
    drafts = [rng.dirichlet(np.ones(V)).astype(np.float32) for _ in range(k)]
    for c in range(1, T):
        q[:, c] = drafts[c - 1]
        qq = drafts[c - 1].astype(np.float64)
        tokens[:, c] = rng.choice(V, size=rows, p=qq / qq.sum())
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (rows, 1))
    u = rng.random((rows, T), dtype=np.float32)
    n = np.full(rows, T, np.int32)
    res = tv.accept_sample(torch.from_numpy(logits).cuda(), 1.0, torch.from_numpy(q).cuda(),
                           torch.from_numpy(u).cuda(), torch.from_numpy(tokens).cuda(),
                           torch.from_numpy(parent).cuda(), torch.from_numpy(n).cuda())
    al, path, bonus = (r.cpu().numpy() for r in res[:3])
    first = np.where(al >= 1, tokens[np.arange(rows), np.maximum(path[:, 1], 0)], bonus)
    p = oracle.sample_probs(root, np.float32(1.0))
    pval = scipy.stats.chisquare(np.bincount(first, minlength=V), p * rows).pvalue
    assert pval > 1e-3


# ----------------------------------------------------------- HIP graphs ---

# ---------------------------------------------------------- draft blocks ---

@pytest.mark.parametrize("T", [1, 16, 33, 100, 128])
@pytest.mark.parametrize("mode", [0, 1])
def test_block_mask_matches_oracle(T, mode):
    n = np.array([T, 0, T // 2, 1, -1, T + 1, max(T - 1, 0)], dtype=np.int32)
    d = torch.from_numpy(n).to(torch.device("cuda:0"))
    mask, pos, st = tv.build_block_mask(d, T, mode)
    torch.cuda.synchronize()
    m_ref, p_ref, s_ref = oracle.build_block_mask(n, T, mode)
    assert np.array_equal(st.cpu().numpy(), s_ref)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), m_ref)
    assert np.array_equal(pos.cpu().numpy(), p_ref)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("chunk", [256, 0])
def test_attention_draft_blocks(mode, chunk):
    # A verification block of 16 rows per sequence (one padded sequence)
    # over ragged contexts: causal (linear draft) or bidirectional (the
    # DFlash block attention). The attention kernel is the tree kernel fed
    # with the block mask.
    w = make_custom(141 + mode, 4, 28, 4, 128, 50, "bf16", [1500, 600, 0, 2047], 15,
                    tree="chain", trie_tokens=False, padded_rows=[1])
    d = upload(w)
    mask, pos, st = tv.build_block_mask(d["n_nodes"], w.T, mode)
    torch.cuda.synchronize()
    m_host = mask.cpu().numpy().view(np.uint32)
    got = run_attention(w, d, mask, chunk_keys=chunk)
    want = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, m_host, w.scale,
                                   max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    check_attention(w, got, want, label="block mode %d" % mode)


@pytest.mark.parametrize("seed", range(19000, 19012))
def test_attention_draft_blocks_random(seed):
    # Seeded draft blocks: block length, batch, ragged contexts (some empty),
    # head grouping, head_dim, causal or bidirectional, probability parts and
    # chunking, against the oracle's masked attention.
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    nd = int(rng.integers(0, 40))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 8))
    D = int(rng.choice([64, 128]))
    ctx = [0 if rng.random() < 0.2 else int(rng.integers(1, 3000)) for _ in range(B)]
    mode = int(rng.integers(0, 2))
    parts = int(rng.choice([2, 3]))
    chunk = int(rng.choice([0, 0, 64, 256]))
    w = make_custom(seed, B, Hkv * G, Hkv, D, 50, "bf16", ctx, nd, tree="chain",
                    trie_tokens=False, padded_rows=[b for b in range(B) if rng.random() < 0.15])
    d = upload(w)
    mask, pos, st = tv.build_block_mask(d["n_nodes"], w.T, mode)
    torch.cuda.synchronize()
    m_host = mask.cpu().numpy().view(np.uint32)
    got = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
    want = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, m_host, w.scale,
                                   max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    check_attention(w, got, want, label="block seed %d mode %d parts %d chunk %d"
                    % (seed, mode, parts, chunk))


# ------------------------------------------------------ few-row projections ---

def _bf16_dev(a):
    from oracle.linear import bf16_bits
    bits = bf16_bits(oracle.round_bf16(a))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.device("cuda:0")), bits


def _linear_bound(x_bits, w_bits, K):
    """Accumulation part of the bound: 2 K 2^-24 sum |x w| (fp32 sums of K
    terms in any order, with slack); the output rounding adds 2^-8 |exact|
    (unit roundoff of bfloat16's 8-bit significand)."""
    xf = np.abs(decode(x_bits, "bf16"))
    wf = np.abs(decode(w_bits, "bf16"))
    return 2.0 * K * 2.0 ** -24 * (xf @ wf.T)


@pytest.mark.parametrize("M,K,N", [(1, 64, 64), (7, 192, 256), (65, 320, 128), (130, 128, 384),
                                   (200, 704, 192), (264, 3584, 4608)])
def test_linear_rows_parity(M, K, N):
    rng = np.random.default_rng(M + K + N)
    x, xb = _bf16_dev(rng.normal(size=(M, K)))
    w, wb = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    y = tv.linear_rows(x, w)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    exact, _ = oracle.linear_rows(xb, wb)
    tol = 2.0 ** -8 * np.abs(exact) + _linear_bound(xb, wb, K) + 1e-30
    assert (np.abs(yg - exact) <= tol).all(), np.abs(yg - exact).max()


def test_linear_rows_batch_invariant():
    # A row's bits depend neither on the row count nor on its place in the
    # batch (sequential K order, no split-K, whatever the tile).
    rng = np.random.default_rng(5)
    M, K, N = 264, 3584, 4608
    x, _ = _bf16_dev(rng.normal(size=(M, K)))
    w, _ = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    full = tv.linear_rows(x, w).cpu().view(torch.int16).numpy()
    for lo, hi in ((0, 1), (5, 71), (100, 264), (263, 264)):
        part = tv.linear_rows(x[lo:hi].contiguous(), w).cpu().view(torch.int16).numpy()
        assert np.array_equal(part, full[lo:hi]), (lo, hi)
    perm = torch.from_numpy(rng.permutation(M)).to(x.device)
    shuffled = tv.linear_rows(x[perm].contiguous(), w).cpu().view(torch.int16).numpy()
    assert np.array_equal(shuffled, full[perm.cpu().numpy()])
    # Strided input rows (a view into a wider buffer) give the same bits.
    wide = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=x.device)
    wide[:, 32:32 + K] = x
    assert np.array_equal(tv.linear_rows(wide[:, 32:32 + K], w).cpu().view(torch.int16).numpy(),
                          full)


def test_linear_batch_invariant_across_tilings():
    # N = 18944 (1184 tiles of 16 features): 193..272 rows run the kernel that
    # keeps every row in each workgroup, fewer rows the 96-row groups; the
    # bits of a row do not change between them (same MFMA chains, k in order).
    rng = np.random.default_rng(9)
    M, K, N = 264, 512, 18944
    x, _ = _bf16_dev(rng.normal(size=(M, K)))
    wg, _ = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    wu, _ = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    full_l = tv.linear_rows(x, wg).cpu().view(torch.int16).numpy()
    full_s = tv.linear_swiglu_rows(x, wg, wu).cpu().view(torch.int16).numpy()
    for lo, hi in ((0, 1), (0, 192), (40, 233), (70, 264), (263, 264)):
        xs = x[lo:hi].contiguous()
        assert np.array_equal(tv.linear_rows(xs, wg).cpu().view(torch.int16).numpy(),
                              full_l[lo:hi]), (lo, hi)
        assert np.array_equal(tv.linear_swiglu_rows(xs, wg, wu).cpu().view(torch.int16).numpy(),
                              full_s[lo:hi]), (lo, hi)


@pytest.mark.parametrize("seed", range(15000, 15016))
def test_linear_rows_random_shapes(seed):
    # Seeded shapes (any row count up to 300, K and N any multiple of 64):
    # the oracle bound, the bits of a random row subset, and the fused SwiGLU
    # against the rounded product of the two projections.
    rng = np.random.default_rng(seed)
    M = int(rng.choice([int(rng.integers(1, 20)), int(rng.integers(20, 300))]))
    K = 64 * int(rng.integers(1, 65))
    N = 64 * int(rng.integers(1, 130))
    x, xb = _bf16_dev(rng.normal(size=(M, K)))
    w, wb = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    y = tv.linear_rows(x, w)
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy().astype(np.float64)
    exact, _ = oracle.linear_rows(xb, wb)
    tol = 2.0 ** -8 * np.abs(exact) + _linear_bound(xb, wb, K) + 1e-30
    assert (np.abs(yg - exact) <= tol).all(), np.abs(yg - exact).max()
    lo = int(rng.integers(0, M))
    hi = int(rng.integers(lo + 1, M + 1))
    part = tv.linear_rows(x[lo:hi].contiguous(), w).cpu().view(torch.int16).numpy()
    assert np.array_equal(part, y.cpu().view(torch.int16).numpy()[lo:hi]), (lo, hi)
    if rng.random() < 0.5:
        wu, _ = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
        ys = tv.linear_swiglu_rows(x, w, wu).float().cpu().numpy().astype(np.float64)
        u = tv.linear_rows(x, wu).float().cpu().numpy().astype(np.float64)
        ref = oracle.round_bf16(oracle.silu(yg) * u)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(ys - ref) <= ulp).all()


@pytest.mark.parametrize("M,K,N", [(9, 64, 64), (100, 448, 320), (264, 3584, 1024),
                                   (264, 3584, 18944)])
def test_linear_swiglu_rows(M, K, N):
    rng = np.random.default_rng(7 * M + K)
    x, xb = _bf16_dev(rng.normal(size=(M, K)))
    wg, wgb = _bf16_dev(rng.normal(size=(N, K)) * 2.0 / np.sqrt(K))
    wu, wub = _bf16_dev(rng.normal(size=(N, K)) / np.sqrt(K))
    y = tv.linear_swiglu_rows(x, wg, wu).float().cpu().numpy().astype(np.float64)
    g = tv.linear_rows(x, wg).float().cpu().numpy().astype(np.float64)
    u = tv.linear_rows(x, wu).float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    # The fused epilogue equals the rounded SwiGLU of the two projections
    # (the same accumulation chains), up to the last bit of fp32 exp.
    ref = oracle.round_bf16(oracle.silu(g) * u)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    diff = np.abs(y - ref)
    assert (diff <= ulp).all(), diff.max()
    assert np.mean(diff == 0) > 0.99
    # And the projections themselves against the oracle bound.
    for got, wb in ((g, wgb), (u, wub)):
        exact, _ = oracle.linear_rows(xb, wb)
        tol = 2.0 ** -8 * np.abs(exact) + _linear_bound(xb, wb, K) + 1e-30
        assert (np.abs(got - exact) <= tol).all()


# ------------------------------------------------------------ KV commit ---

def _bits(t):
    """Raw element bits of a device tensor (NaN payloads compared too)."""
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy()
    return a.view(torch.int32).numpy()


def _commit_case(w, k_host, v_host, acc, path, layers_first=False):
    """Commit on the GPU (caches as given) and with the oracle; compare bits."""
    dev_ = torch.device("cuda:0")
    conv = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev_)) if w.dtype == "bf16" else (lambda a: torch.from_numpy(
            np.ascontiguousarray(a)).to(dev_))
    k, v = conv(k_host), conv(v_host)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev_)
    ctx, n = i32(w.ctx_len), i32(w.n_nodes)
    new_ctx, st = tv.commit_accepted_kv(k, v, ctx, n, i32(acc), i32(path))
    torch.cuda.synchronize()
    kr, vr, ctx_r, st_r = oracle.commit_accepted_kv(k_host, v_host, w.ctx_len, w.n_nodes, acc, path)
    assert np.array_equal(st.cpu().numpy(), st_r), (st.cpu().numpy(), st_r)
    assert np.array_equal(new_ctx.cpu().numpy(), ctx_r)
    dt = np.int16 if w.dtype == "bf16" else np.int32
    assert np.array_equal(_bits(k), np.ascontiguousarray(kr).view(dt))
    assert np.array_equal(_bits(v), np.ascontiguousarray(vr).view(dt))
    return st_r


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_commit_after_greedy_acceptance(name):
    # The path and accept_len come from the GPU acceptance of the same tree.
    w = make_config(name)
    d = upload(w)
    al, path, _, _, st = run_greedy(d)
    assert not st.any()
    st_c = _commit_case(w, w.k, w.v, al, path)
    assert not st_c.any()


@pytest.mark.parametrize("seed", range(17000, 17012))
def test_commit_random_paths(seed):
    # Seeded trees, contexts and element types; each live sequence accepts the
    # root-to-node path of a random node (any depth, the root alone included).
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    D = int(rng.choice([64, 128]))
    ctx = [int(rng.integers(0, 700)) for _ in range(B)]
    nd = int(rng.integers(0, 100))
    w = make_custom(seed, B, 4, 2, D, 50, dtype, ctx, nd, trie_tokens=False,
                    padded_rows=[b for b in range(B) if rng.random() < 0.15])
    T = w.T
    path = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        n = int(w.n_nodes[b])
        if n == 0:
            continue
        node = int(rng.integers(0, n))
        chain = [node]
        while chain[-1] != 0:
            chain.append(int(w.parent[b, chain[-1]]))
        chain = chain[::-1]
        path[b, :len(chain)] = chain
        acc[b] = len(chain) - 1
    st = _commit_case(w, w.k, w.v, acc, path)
    assert not st.any()


def test_commit_layers_nhd_fp32_and_long_paths():
    # Three layers of an fp32 cache laid out [layer][B][capacity][Hkv][D]
    # (NHD) and seen through strides; a chain of 128 rows whose path skips
    # node 1 (slot L+k takes slot L+k+1: every source but the last is the
    # next destination) across several 16-row batches; a bushy tree.
    w = make_custom(91, 3, 8, 2, 64, 50, "f32", [300, 0, 41], 127, tree="chain",
                    trie_tokens=False)
    T = w.T
    path = np.full((w.B, T), -1, np.int32)
    acc = np.zeros(w.B, np.int32)
    path[0, 0] = 0
    path[0, 1:T - 1] = np.arange(2, T)
    acc[0] = T - 2
    path[1, :T] = np.arange(T)
    acc[1] = T - 1
    path[2, :3] = [0, 1, 2]
    acc[2] = 2
    rng = np.random.default_rng(2)
    layers = 3
    kl = np.stack([w.k + np.float32(10 * l) for l in range(layers)])
    vl = np.stack([w.v - np.float32(10 * l) for l in range(layers)])
    dev_ = torch.device("cuda:0")
    # NHD storage, viewed as [layer][B][Hkv][capacity][D].
    k_nhd = torch.from_numpy(np.ascontiguousarray(kl.transpose(0, 1, 3, 2, 4))).to(dev_)
    v_nhd = torch.from_numpy(np.ascontiguousarray(vl.transpose(0, 1, 3, 2, 4))).to(dev_)
    k = k_nhd.permute(0, 1, 3, 2, 4)
    v = v_nhd.permute(0, 1, 3, 2, 4)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev_)
    new_ctx, st = tv.commit_accepted_kv(k, v, i32(w.ctx_len), i32(w.n_nodes), i32(acc), i32(path))
    torch.cuda.synchronize()
    kr, vr, ctx_r, st_r = oracle.commit_accepted_kv(kl, vl, w.ctx_len, w.n_nodes, acc, path)
    assert not st_r.any()
    assert np.array_equal(st.cpu().numpy(), st_r) and np.array_equal(new_ctx.cpu().numpy(), ctx_r)
    assert np.array_equal(k.cpu().numpy().view(np.int32), kr.view(np.int32))
    assert np.array_equal(v.cpu().numpy().view(np.int32), vr.view(np.int32))
    del rng


def test_commit_status_and_untouched_sequences():
    w = make_custom(93, 5, 4, 2, 128, 50, "bf16", [64, 10, 20, 30, 5], 9, padded_rows=[4],
                    trie_tokens=False)
    T = w.T
    path = np.full((w.B, T), -1, np.int32)
    acc = np.zeros(w.B, np.int32)
    # 0: valid two-step path; 1: not increasing; 2: accept_len too long;
    # 3: path[0] != 0; 4: padded sequence.
    p0 = oracle.ancestors(w.parent[0], int(w.n_nodes[0]) - 1)[::-1]
    path[0, :len(p0)] = p0
    acc[0] = len(p0) - 1
    path[1, :3] = [0, 2, 1]
    acc[1] = 2
    acc[2] = int(w.n_nodes[2])
    path[2, :T] = np.arange(T)
    path[3, :2] = [1, 2]
    acc[3] = 1
    st = _commit_case(w, w.k, w.v, acc, path)
    assert list(st) == [0, oracle.ROW_BAD_PATH, oracle.ROW_BAD_PATH, oracle.ROW_BAD_PATH, 0]


# --------------------------------------------------------- packed rows ---

def _packed_layout(w, seed, gap=3):
    """Row starts for the live rows of w in a shuffled sequence order with a
    few spare rows between sequences, and q packed accordingly."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(w.B)
    start = np.zeros(w.B, np.int32)
    pos = 1
    for b in order:
        start[b] = pos
        pos += int(w.n_nodes[b]) + int(rng.integers(0, gap + 1))
    rows = pos + 2
    qp = np.zeros((rows,) + w.q.shape[2:], w.q.dtype)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        qp[start[b]:start[b] + n] = w.q[b, :n]
    return qp, start, rows


def _run_packed(w, d, mask, qp, start, chunk=0, parts=3, sentinel=12345.0):
    qd = torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).cuda() if w.dtype == "bf16" \
        else torch.from_numpy(qp).cuda()
    rows = qp.shape[0]
    out = torch.full((rows, w.Hq, w.D), sentinel, dtype=torch.float32, device="cuda")
    lse = torch.full((rows, w.Hq), sentinel, dtype=torch.float32, device="cuda")
    st_d = torch.from_numpy(start).cuda()
    o, l, st = tv.tree_attention_packed(qd, d["k"], d["v"], d["ctx_len"], d["n_nodes"], mask,
                                        st_d, w.max_ctx, scale=float(w.scale),
                                        probability_parts=parts, chunk_keys=chunk, out=out,
                                        lse=lse)
    torch.cuda.synchronize()
    return o.cpu().numpy(), l.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("name,chunk,parts", [("C3", 0, 3), ("C3", 512, 3), ("C2", 0, 3),
                                              ("C1", 0, 3), ("C3", 0, 1)])
def test_attention_packed_bitwise_equals_padded(name, chunk, parts):
    # The packed launch keeps the padded launch's split partition, so every
    # live row carries exactly the padded call's bits; spare rows between the
    # sequences keep what they held.
    w = make_config(name)
    d = upload(w)
    mask = _mask_check(w, d)
    o_pad, l_pad, st_pad = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
    qp, start, rows = _packed_layout(w, 5)
    o, l, st = _run_packed(w, d, mask, qp, start, chunk=chunk, parts=parts)
    assert np.array_equal(st, st_pad)
    owned = np.zeros(rows, bool)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        s0 = int(start[b])
        owned[s0:s0 + n] = True
        assert np.array_equal(o[s0:s0 + n].view(np.uint32), o_pad[b, :n].view(np.uint32)), b
        assert np.array_equal(l[s0:s0 + n].view(np.uint32), l_pad[b, :n].view(np.uint32)), b
    assert np.all(o[~owned] == 12345.0) and np.all(l[~owned] == 12345.0)
    # And against the oracle over packed rows.
    o_ref, l_ref, st_ref = oracle.tree_attention_packed(
        qp, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, w.parent, start, w.T, w.scale,
        max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    assert np.array_equal(st, st_ref)
    live = ~np.isnan(l_ref)
    assert np.array_equal(live, owned[:, None] & np.ones((1, w.Hq), bool))
    assert np.abs(o[live] - o_ref[live]).max() <= 2e-3
    assert np.abs(l[live] - l_ref[live]).max() <= 1e-4


def _random_case(seed, bmax, ctxmax, ndmax):
    """One seeded draw over the attention call's parameters: head_dim,
    input type, group size, batch, ragged contexts (some empty), tree size
    and shape, padded sequences, probability parts, chunking and the packed
    layout."""
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 8))
    B = int(rng.integers(1, bmax))
    ctx = [0 if rng.random() < 0.1 else int(rng.integers(1, ctxmax)) for _ in range(B)]
    nd = int(rng.integers(0, ndmax))
    tree = str(rng.choice(["random", "random", "chain", "star"]))
    padded = [b for b in range(B) if rng.random() < 0.15]
    parts = int(rng.choice([1, 2, 3, 3])) if dtype == "bf16" else 3
    chunk = int(rng.choice([0, 0, 0, 64, 128, 512]))
    packed = bool(rng.random() < 0.3)
    w = make_custom(seed, B, Hkv * G, Hkv, D, 64, dtype, ctx, nd, tree=tree, padded_rows=padded,
                    trie_tokens=False)
    return w, parts, chunk, packed


@pytest.mark.parametrize("seed,bmax,ctxmax,ndmax",
                         [(7000 + i, 7, 2500, 48) for i in range(40)] +
                         [(9000 + i, 90, 1500, 128) for i in range(12)])
def test_attention_random_cases(seed, bmax, ctxmax, ndmax):
    # Seeded random draws over the whole parameter space, up to 89 sequences
    # (more pairs than workgroups: the stream-K partition) and 128-row trees,
    # each against the oracle at the bound of its probability parts.
    w, parts, chunk, packed = _random_case(seed, bmax, ctxmax, ndmax)
    d = upload(w)
    mask = tv.build_tree_mask(d["parent"], d["n_nodes"])[0]
    atol = fast_mode_bound(w) if parts == 1 else ATOL_OUT
    if not packed:
        got = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
        check_attention(w, got, oracle_attention(w), atol_out=atol,
                        label="seed %d parts %d chunk %d" % (seed, parts, chunk))
        return
    qp, start, rows = _packed_layout(w, 3)
    o, l, st = _run_packed(w, d, mask, qp, start, chunk=chunk, parts=parts)
    o_ref, l_ref, st_ref = oracle.tree_attention_packed(
        qp, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, w.parent, start, w.T, w.scale,
        max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    assert np.array_equal(st, st_ref)
    live = ~np.isnan(l_ref)
    assert np.all(o[~live] == 12345.0) and np.all(l[~live] == 12345.0)
    fin = live & np.isfinite(l_ref)
    assert np.array_equal(l[live & ~fin], l_ref[live & ~fin])
    err_o = float(np.abs(o[live] - o_ref[live]).max(initial=0.0))
    err_l = float(np.abs(l[fin] - l_ref[fin]).max(initial=0.0))
    print("packed seed %d parts %d chunk %d: max|out - oracle| = %.3g, max|lse - oracle| = %.3g"
          % (seed, parts, chunk, err_o, err_l))
    assert err_o <= atol and err_l <= 1e-4


@pytest.mark.parametrize("dtype,D,chunk", [("f32", 64, 128), ("bf16", 64, 0), ("bf16", 128, 64)])
def test_attention_packed_ragged_and_statuses(dtype, D, chunk):
    # Ragged trees and contexts, G = 3; one sequence over its context bound
    # (its own rows get 0 / -inf), one with a start past the rows (nothing
    # written), one padded (nothing written).
    w = make_custom(77 + D, 6, 9, 3, D, 50, dtype, [300, 0, 77, 1000, 129, 64], 20,
                    n_nodes=[21, 21, 13, 0, 1, 9], trie_tokens=False)
    d = upload(w)
    mask = _mask_check(w, d)
    qp, start, rows = _packed_layout(w, 9)
    ctx = w.ctx_len.copy()
    ctx[4] = w.max_ctx + 1                      # context bound
    start[5] = rows - 3                         # 9 rows do not fit
    d["ctx_len"] = torch.from_numpy(ctx.astype(np.int32)).cuda()
    o, l, st = _run_packed(w, d, mask, qp, start, chunk=chunk)
    o_ref, l_ref, st_ref = oracle.tree_attention_packed(
        qp, w.k, w.v, w.dtype, ctx, w.n_nodes, w.parent, start, w.T, w.scale,
        max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    assert st.tolist() == st_ref.tolist()
    assert st_ref[4] == oracle.ROW_CTX_BOUND and st_ref[5] == oracle.ROW_BAD_START
    untouched = np.isnan(l_ref)
    assert np.all(l[untouched] == 12345.0) and np.all(o[untouched] == 12345.0)
    live = ~untouched
    assert not np.isnan(o[live]).any()
    err = np.abs(o[live] - o_ref[live]).max()
    print("packed ragged: max|out - oracle| = %.3g" % err)
    assert err <= ATOL_OUT
    dead = live & (l_ref == -np.inf)            # the context-bound sequence's rows
    assert dead.sum() == int(w.n_nodes[4]) * w.Hq and np.all(l[dead] == -np.inf)
    fin = live & ~dead
    assert np.abs(l[fin] - l_ref[fin]).max() <= 1e-4


# ------------------------------------------------------- adaptive budget ---

def _budget_gpu(acc, n, ema, bud, target, alpha, n_min, n_max, status=None):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dt)).cuda()
    ema_d = t(ema, np.float32)
    bud_d = t(bud, np.int32)
    st_d = None if status is None else t(status, np.int32)
    start, total = tv.adapt_tree_budget(t(acc, np.int32), t(n, np.int32), ema_d, bud_d, target,
                                        alpha, n_min, n_max, row_status=st_d)
    torch.cuda.synchronize()
    return (ema_d.cpu().numpy(), bud_d.cpu().numpy(), start.cpu().numpy(),
            int(total.cpu().numpy()[0]))


def test_budget_golden_trajectory(golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "budget_hand.json")) as f:
        g = json.load(f)
    ema = np.array(g["ema0"], np.float32)
    bud = np.array(g["budget0"], np.int32)
    for step in g["steps"]:
        ema, bud, start, total = _budget_gpu(step["accept_len"], step["n_nodes"], ema, bud,
                                             g["target"], g["alpha"], g["n_min"], g["n_max"],
                                             step["row_status"])
        assert ema.tolist() == step["ema"] and bud.tolist() == step["budget"], step["why"]
        assert start.tolist() == step["row_start"] and total == step["rows_total"]


@pytest.mark.parametrize("B", [1, 64, 1000, 3000])
def test_budget_matches_oracle_bitwise(B):
    # Random acceptance over 25 steps (invalid lengths, bad statuses, padded
    # and root-only steps included); float32 state and budgets bit for bit.
    rng = np.random.default_rng(B)
    target, alpha, n_min, n_max = 0.37, 0.2, 2, 100
    ema_g = ema_o = rng.random(B).astype(np.float32)
    bud_g = bud_o = rng.integers(n_min, n_max + 1, B).astype(np.int32)
    for step in range(25):
        n = np.minimum(bud_o + 1, 128).astype(np.int32)
        n[rng.random(B) < 0.05] = 0
        n[rng.random(B) < 0.05] = 1
        acc = (rng.random(B) * n).astype(np.int32)
        acc[rng.random(B) < 0.02] = 200
        status = (rng.random(B) < 0.03).astype(np.int32) * 2
        ema_g, bud_g, start_g, tot_g = _budget_gpu(acc, n, ema_g, bud_g, target, alpha, n_min,
                                                   n_max, status)
        ema_o, bud_o, start_o, tot_o = oracle.adapt_tree_budget(acc, n, ema_o, bud_o, target,
                                                                alpha, n_min, n_max, status)
        assert np.array_equal(ema_g.view(np.uint32), ema_o.view(np.uint32)), step
        assert np.array_equal(bud_g, bud_o) and np.array_equal(start_g, start_o), step
        assert tot_g == tot_o


def test_budget_empty_batch():
    ema, bud, start, total = _budget_gpu(np.zeros(0), np.zeros(0), np.zeros(0), np.zeros(0),
                                         0.5, 0.5, 1, 8)
    assert total == 0 and start.size == 0


def test_graph_capture_replays_match_eager():
    w = make_config("C2")
    d = upload(w)
    mask_e, _, _ = tv.build_tree_mask(d["parent"], d["n_nodes"])
    out_e, lse_e, _ = tv.tree_attention(d["q"], d["k"], d["v"], d["ctx_len"], d["n_nodes"],
                                        mask_e, w.max_ctx, scale=float(w.scale))
    acc_e = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
    torch.cuda.synchronize()
    ref = [out_e.cpu(), lse_e.cpu()] + [a.cpu() for a in acc_e]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g):
            mask, _, _ = tv.build_tree_mask(d["parent"], d["n_nodes"])
            out, lse, _ = tv.tree_attention(d["q"], d["k"], d["v"], d["ctx_len"], d["n_nodes"],
                                            mask, w.max_ctx, scale=float(w.scale))
            acc = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(7.0)
        acc[0].fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [out.cpu(), lse.cpu()] + [a.cpu() for a in acc]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep


def test_graph_capture_whole_step_with_next_rows():
    # One captured step over every other entry point: block masks, packed
    # attention, greedy acceptance, KV commit, the budget controller and a
    # projection. The commit and the controller update state in place, so the
    # state is restored (outside the graph) before each replay; every replay
    # must reproduce the eager results bit for bit.
    w = make_config("C2")
    d = upload(w)
    qp, start, rows = _packed_layout(w, 11)
    qd = torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).cuda()
    start_d = torch.from_numpy(start).cuda()
    g = torch.Generator().manual_seed(5)
    x = torch.randn(w.B * w.T, 256, generator=g).to(torch.bfloat16).cuda()
    wt = torch.randn(128, 256, generator=g).to(torch.bfloat16).cuda()
    k0, v0 = d["k"].clone(), d["v"].clone()
    ema0 = torch.full((w.B,), 0.5, dtype=torch.float32, device="cuda")
    bud0 = torch.full((w.B,), w.T - 1, dtype=torch.int32, device="cuda")
    k, v, ema, bud = k0.clone(), v0.clone(), ema0.clone(), bud0.clone()

    def step():
        bm, pos, _ = tv.build_block_mask(d["n_nodes"], w.T, tv.TV_BLOCK_CAUSAL)
        mask, _, _ = tv.build_tree_mask(d["parent"], d["n_nodes"])
        o, l, _ = tv.tree_attention_packed(qd, k, v, d["ctx_len"], d["n_nodes"], mask, start_d,
                                           w.max_ctx, scale=float(w.scale))
        acc = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
        new_ctx, _ = tv.commit_accepted_kv(k, v, d["ctx_len"], d["n_nodes"], acc[0], acc[1])
        rs, rt = tv.adapt_tree_budget(acc[0], d["n_nodes"], ema, bud, 0.6, 0.25, 2, 64)
        y = tv.linear_rows(x, wt)
        return [bm, pos, o, l] + list(acc) + [new_ctx, rs, rt, y]

    owned = torch.zeros(rows, dtype=torch.bool)
    for b in range(w.B):
        owned[int(start[b]):int(start[b]) + int(w.n_nodes[b])] = True
    eager = step()
    torch.cuda.synchronize()
    ref = [t.cpu() for t in eager] + [k.cpu(), v.cpu(), ema.cpu(), bud.cpu()]

    k.copy_(k0); v.copy_(v0); ema.copy_(ema0); bud.copy_(bud0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph):
            outs = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        k.copy_(k0); v.copy_(v0); ema.copy_(ema0); bud.copy_(bud0)
        for t in outs:
            t.fill_(3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in outs] + [k.cpu(), v.cpu(), ema.cpu(), bud.cpu()]
        for i, (a, b) in enumerate(zip(got, ref)):
            if i in (2, 3):  # packed out / lse: only the sequences' own rows are written
                a, b = a[owned], b[owned]
            assert torch.equal(_raw_bits(a), _raw_bits(b)), (rep, i)


def _raw_bits(t):
    # Raw bits of a host tensor, so that NaN (dead cache slots) equals itself.
    if t.is_floating_point():
        return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])
    return t


# ------------------------------------------------------- more than 64 seqs ---

def _many_seqs(seed, dtype, B=150):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, 400, B)
    n = rng.integers(1, 10, B)
    n[rng.random(B) < 0.1] = 0          # padded sequences, also past 64
    return make_custom(seed, B, 4, 2, 64, 50, dtype, ctx.tolist(), 8, n_nodes=n.tolist(),
                       trie_tokens=False)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 0), ("bf16", 128), ("f32", 0)])
def test_attention_more_than_64_sequences(dtype, chunk):
    # Sequences past the first 64 take the block-scan paths of the schedule
    # (unit size, unit decode, the combine's table) and the memory loads of
    # their lengths; one of them is over its context bound.
    w = _many_seqs(300 + chunk, dtype)
    w.ctx_len[100] = w.max_ctx + 5 if w.n_nodes[100] else w.ctx_len[100]
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=chunk)
    check_attention(w, got, oracle_attention(w), label="%d sequences" % w.B)


def test_attention_packed_more_than_64_sequences():
    w = _many_seqs(401, "bf16")
    d = upload(w)
    mask = _mask_check(w, d)
    qp, start, rows = _packed_layout(w, 13)
    ctx = w.ctx_len.copy()
    live_late = [b for b in range(70, w.B) if w.n_nodes[b] > 0]
    ctx[live_late[0]] = w.max_ctx + 1          # context bound past 64
    start[live_late[1]] = rows                 # start past the rows, past 64
    d["ctx_len"] = torch.from_numpy(ctx.astype(np.int32)).cuda()
    o, l, st = _run_packed(w, d, mask, qp, start)
    o_ref, l_ref, st_ref = oracle.tree_attention_packed(
        qp, w.k, w.v, w.dtype, ctx, w.n_nodes, w.parent, start, w.T, w.scale,
        max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    assert st.tolist() == st_ref.tolist()
    assert st_ref[live_late[0]] == oracle.ROW_CTX_BOUND
    assert st_ref[live_late[1]] == oracle.ROW_BAD_START
    untouched = np.isnan(l_ref)
    assert np.all(l[untouched] == 12345.0) and np.all(o[untouched] == 12345.0)
    live = ~untouched
    err = np.abs(o[live] - o_ref[live]).max()
    print("packed, %d sequences: max|out - oracle| = %.3g" % (w.B, err))
    assert err <= ATOL_OUT
    fin = live & (l_ref > -np.inf)
    assert np.all(l[live & ~fin] == -np.inf)
    assert np.abs(l[fin] - l_ref[fin]).max() <= 1e-4
    # And bitwise equal to the padded call for every live sequence, given the
    # same live set: the balanced partition spans every live sequence, so
    # the sequence whose packed start is out of bounds (not live here) is
    # made not live in the padded call too (context past its bound).
    ctx_pad = ctx.copy()
    ctx_pad[live_late[1]] = w.max_ctx + 1
    d["ctx_len"] = torch.from_numpy(ctx_pad.astype(np.int32)).cuda()
    o_pad, l_pad, _ = run_attention(w, d, mask)
    for b in range(w.B):
        n = int(w.n_nodes[b])
        if st_ref[b] == 0 and n:
            s0 = int(start[b])
            assert np.array_equal(o[s0:s0 + n].view(np.uint32), o_pad[b, :n].view(np.uint32)), b


# ----------------------------------------------------------- largest trees ---

@pytest.mark.parametrize("dtype,D,chunk", [("bf16", 128, 0), ("bf16", 64, 64), ("f32", 128, 0),
                                           ("f32", 64, 256)])
def test_attention_largest_tree_and_group(dtype, D, chunk):
    # T = TV_MAX_TREE rows and G = TV_MAX_GROUP query heads per KV head:
    # 2048 packed rows per (sequence, KV head), the last one the edge of the
    # row -> node multiplier; several row groups per pair; a full, a partial
    # and a root-only tree over ragged contexts (one empty).
    w = make_custom(501 + D, 3, 16, 1, D, 50, dtype, [700, 0, 129], 127,
                    n_nodes=[128, 100, 1], max_depth=40, trie_tokens=False)
    assert w.T == tv.TV_MAX_TREE and w.Hq // w.Hkv == tv.TV_MAX_GROUP
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=chunk)
    check_attention(w, got, oracle_attention(w), label="T=128, G=16")


def test_greedy_largest_tree():
    w = make_custom(611, 3, 2, 1, 64, 1000, "bf16", [4, 4, 4], 127, n_nodes=[128, 57, 1],
                    max_depth=40, plant_depth=4)
    d = upload(w)
    check_greedy(run_greedy(d), oracle.accept_greedy(w.logits, w.tokens, w.parent, w.n_nodes))


def test_sample_largest_tree():
    w = make_custom(612, 3, 2, 1, 64, 300, "bf16", [4, 4, 4], 127, n_nodes=[128, 90, 1],
                    max_depth=40, mode="sample", temperature=0.9)
    d = upload(w)
    got = run_sample(w, d)
    want = oracle.accept_sample(w.logits, w.temperature, w.qdraft, w.u, w.tokens, w.parent,
                                w.n_nodes)
    check_sample(w, got, want)


def _many_rounds_case(D, parts):
    return make_custom(701 + D + parts, 2, 8, 2, D, 50, "bf16", [1500, 2100], 20,
                       n_nodes=[21, 13], trie_tokens=False)


@pytest.mark.parametrize("D,parts", [(64, 3), (128, 3), (64, 2)])
def test_attention_combine_many_rounds(D, parts):
    # More than 16 units per pair (the combine's per-round batch): 64-key
    # chunks over 1500- and 2100-key contexts give 24 and 33 units, so the
    # merge runs two and three rounds; with D = 64 and one part a lane holds
    # two unit records per round.
    w = _many_rounds_case(D, parts)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=64, parts=parts)
    check_attention(w, got, oracle_attention(w), label="D=%d parts=%d" % (D, parts))


@pytest.mark.parametrize("D", [64, 128])
def test_attention_fast_mode_combine_many_rounds(D):
    # The fast mode's 16-bit partials through a merge of 24 and 33 units.
    w = _many_rounds_case(D, 1)
    d = upload(w)
    mask = _mask_check(w, d)
    got = run_attention(w, d, mask, chunk_keys=64, parts=1)
    check_attention(w, got, oracle_attention(w), atol_out=fast_mode_bound(w), label="fast mode")


# ------------------------------------------------------------ bf16 output ---

def _bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (8-bit significand)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@pytest.mark.parametrize("name,chunk", [("C2", 0), ("C3", 0), ("C1", 0), ("C2", 128)])
def test_attention_bf16_output(name, chunk):
    # out_dtype = bf16: the fp32 result of the same call rounded to nearest
    # even once (bitwise), within one bf16 ulp of the oracle rounded to bf16;
    # lse is fp32 and identical to the fp32-output call.
    w = make_config(name)
    d = upload(w)
    mask = _mask_check(w, d)
    o32, l32, st32 = run_attention(w, d, mask, chunk_keys=chunk)
    ob = tv.tree_attention(d["q"], d["k"], d["v"], d["ctx_len"], d["n_nodes"], mask, w.max_ctx,
                           scale=float(w.scale), chunk_keys=chunk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert ob[0].dtype == torch.bfloat16
    rounded = torch.from_numpy(o32).to(torch.bfloat16)
    assert torch.equal(ob[0].cpu().view(torch.int16), rounded.view(torch.int16))
    assert np.array_equal(ob[1].cpu().numpy().view(np.uint32), l32.view(np.uint32))
    assert np.array_equal(ob[2].cpu().numpy(), st32)
    # |bf16(g) - bf16(x)| <= ulp/2 + |g - x| + ulp/2 for the fp32 result g of
    # the same call and the exact x: within one bf16 ulp of the oracle
    # rounded to bf16, beyond the fp32 result's own (2e-3-bounded) error.
    o_ref, _, _ = oracle_attention(w)
    ref_b = torch.from_numpy(o_ref).to(torch.bfloat16).double().numpy()
    got_b = ob[0].double().cpu().numpy()
    live = np.zeros(l32.shape, bool)
    for b in range(w.B):
        live[b, : int(w.n_nodes[b])] = True
    diff = np.abs(got_b[live] - ref_b[live])
    ulp = np.maximum(_bf16_ulp(ref_b[live]), _bf16_ulp(got_b[live]))
    err32 = np.abs(o32[live] - o_ref[live])
    assert (diff <= ulp + err32).all(), (diff - ulp - err32).max()
    print("bf16 out: %.1f%% of entries equal to the rounded oracle" %
          (100.0 * np.mean(diff == 0)))
    assert np.all(got_b[~live] == 0.0)
    # Packed rows write the same bf16 bits.
    qp, start, rows = _packed_layout(w, 21)
    qd = torch.from_numpy(qp.view(np.int16)).view(torch.bfloat16).cuda() if w.dtype == "bf16" \
        else torch.from_numpy(qp).cuda()
    op, lp, _ = tv.tree_attention_packed(qd, d["k"], d["v"], d["ctx_len"], d["n_nodes"], mask,
                                         torch.from_numpy(start).cuda(), w.max_ctx,
                                         scale=float(w.scale), chunk_keys=chunk,
                                         out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for b in range(w.B):
        n, s0 = int(w.n_nodes[b]), int(start[b])
        assert torch.equal(op[s0:s0 + n].cpu().view(torch.int16),
                           ob[0][b, :n].cpu().view(torch.int16)), b


# ------------------------------------------ rows that see few or no keys ---

def test_attention_explicit_mask_without_first_keys():
    # Caller-built masks over an empty committed context: row 0 sees nothing
    # (out 0, lse -inf), row 35 sees only keys 33 and 35 (none of the unit's
    # first 32 keys, so its reference comes from later keys), row 36 sees all.
    w = make_custom(63, 2, 8, 2, 128, 50, "bf16", [0, 300], 39, tree="chain",
                    trie_tokens=False, padded_rows=[])
    d = upload(w)
    m_host, _, _ = oracle.build_block_mask(w.n_nodes, w.T, oracle.CAUSAL)
    m_host[0, 0] = 0
    m_host[0, 35] = [0, (1 << 1) | (1 << 3)]
    m_host[0, 36] = [0xFFFFFFFF, 0xFF]
    m_host[1, 35] = [0, 1 << 3]          # with committed keys: sees them and key 35
    mask = torch.from_numpy(m_host.view(np.int32)).cuda()
    want = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, m_host, w.scale,
                                   max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    assert np.all(want[1][0, 0] == -np.inf)
    for parts in (3, 2):
        for chunk in (64, 0):
            got = run_attention(w, d, mask, chunk_keys=chunk, parts=parts)
            check_attention(w, got, want, label="parts=%d chunk=%d" % (parts, chunk))
            assert np.all(got[0][0, 0] == 0.0) and np.all(got[1][0, 0] == -np.inf)


# ------------------------------------------------- C3-shaped draft blocks ---

@pytest.mark.parametrize("mode", [0, 1])
def test_attention_draft_blocks_c3_shape(mode):
    # 16-row draft blocks (causal linear drafts, or the bidirectional DFlash
    # block attention) over the headline shapes: 8 sequences, 28/4 heads,
    # D = 128, contexts of 4096-8192 keys, one sequence with no committed
    # context at all; page precision (three parts), balanced and fixed units.
    ctx = [4096, 8192, 0, 5000, 7777, 6143, 4100, 8000]
    w = make_custom(151 + mode, 8, 28, 4, 128, 50, "bf16", ctx, 15, tree="chain",
                    trie_tokens=False, padded_rows=[])
    d = upload(w)
    mask, _, st = tv.build_block_mask(d["n_nodes"], w.T, mode)
    torch.cuda.synchronize()
    m_host = mask.cpu().numpy().view(np.uint32)
    want = oracle.masked_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, m_host, w.scale,
                                   max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)
    for chunk in (0, 512):
        got = run_attention(w, d, mask, chunk_keys=chunk)
        check_attention(w, got, want, label="block mode %d chunk %d" % (mode, chunk))
