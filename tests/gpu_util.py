"""Helpers of the GPU parity tests: upload a workload, run the HIP path,
compare against the float64 oracle at the stated tolerances."""

import numpy as np
import torch

import oracle
from oracle.decode import decode
import tree_attention_draft_tv_amd as tv

# Attention tolerances (max abs error over live entries).
ATOL_OUT = 2e-3
ATOL_LSE = 1e-4
# Sampling: a test whose |u - ratio| is below this is exempt from bit-exactness.
SAMPLE_BAND = 1e-6


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def qkv_to_dev(w):
    if w.dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev())
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return conv(w.q), conv(w.k), conv(w.v)


def upload(w):
    d = {}
    d["q"], d["k"], d["v"] = qkv_to_dev(w)
    d["ctx_len"] = to_dev(w.ctx_len.astype(np.int32))
    d["n_nodes"] = to_dev(w.n_nodes.astype(np.int32))
    d["parent"] = to_dev(w.parent.astype(np.int32))
    d["tokens"] = to_dev(w.tokens.astype(np.int32))
    if w.logits is not None:
        d["logits"] = to_dev(w.logits)
    if w.qdraft is not None:
        d["qdraft"] = to_dev(w.qdraft)
        d["u"] = to_dev(w.u)
    return d


def run_mask(d, T):
    mask, depth, status = tv.build_tree_mask(d["parent"], d["n_nodes"])
    return mask, depth, status


def run_attention(w, d, mask, chunk_keys=0, parts=3, max_ctx=None, out_dtype=torch.float32):
    out, lse, st = tv.tree_attention(d["q"], d["k"], d["v"], d["ctx_len"], d["n_nodes"], mask,
                                     w.max_ctx if max_ctx is None else max_ctx,
                                     scale=float(w.scale), probability_parts=parts,
                                     chunk_keys=chunk_keys, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), st.cpu().numpy()


def oracle_attention(w):
    return oracle.tree_attention(w.q, w.k, w.v, w.dtype, w.ctx_len, w.n_nodes, w.parent,
                                 w.scale, max_ctx=w.max_ctx, kv_capacity=w.kv_capacity)


def fast_mode_bound(w):
    """Error bound of the lossy fast mode (probability_parts = 1), as
    include/tv.h states it: each probability rounded once to bf16 (relative
    error <= 2^-8, the unit roundoff of an 8-bit significand) and the split
    partials kept as 16-bit fixed point (<= max|v| / 65534), so an output
    entry is within (2^-8 + 2^-16) max|v| over the visible values, plus fp32
    accumulation slack. Only tests of that mode use it; every other
    attention test holds the 2e-3 / 1e-4 bound."""
    vmax = 0.0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        if n:
            live = decode(w.v[b, :, : int(w.ctx_len[b]) + n], w.dtype)
            vmax = max(vmax, float(np.abs(live).max()))
    return max(ATOL_OUT, (2.0 ** -8 + 2.0 ** -16) * vmax + 1e-5)


def check_attention(w, got, want, atol_out=ATOL_OUT, atol_lse=ATOL_LSE, label=""):
    """Statuses equal, no NaN, live entries within the bounds (max abs error),
    padding exactly 0 / -inf. Prints and returns (err_out, err_lse)."""
    out, lse, st = got
    o_ref, l_ref, st_ref = want
    assert np.array_equal(st, st_ref), (st, st_ref)
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    live = np.zeros(lse.shape, bool)
    for b in range(w.B):
        if st_ref[b] == 0:
            live[b, : int(w.n_nodes[b])] = True
    err_o = float(np.abs(out[live] - o_ref[live]).max(initial=0.0))
    fin = live & np.isfinite(l_ref)
    assert np.array_equal(lse[live & ~fin], l_ref[live & ~fin])  # rows that see no key
    err_l = float(np.abs(lse[fin] - l_ref[fin]).max(initial=0.0))
    print("attention %s: max|out - oracle| = %.3g (bound %.3g), max|lse - oracle| = %.3g "
          "(bound %.3g)" % (label, err_o, atol_out, err_l, atol_lse))
    assert err_o <= atol_out, "max |out - oracle| = %g" % err_o
    assert err_l <= atol_lse, "max |lse - oracle| = %g" % err_l
    assert np.all(out[~live] == 0.0)
    assert np.all(lse[~live] == -np.inf)
    return err_o, err_l


def run_greedy(d):
    res = tv.accept_greedy(d["logits"], d["tokens"], d["parent"], d["n_nodes"])
    torch.cuda.synchronize()
    return tuple(r.cpu().numpy() for r in res)


def check_greedy(got, want):
    al, path, bonus, am, st = got
    al_r, path_r, bonus_r, am_r, st_r = want
    assert np.array_equal(st, st_r), (st, st_r)
    assert np.array_equal(al, al_r), (al, al_r)
    assert np.array_equal(path, path_r)
    assert np.array_equal(bonus, bonus_r), (bonus, bonus_r)
    assert np.array_equal(am, am_r)


def run_sample(w, d):
    res = tv.accept_sample(d["logits"], float(w.temperature), d["qdraft"], d["u"], d["tokens"],
                           d["parent"], d["n_nodes"])
    torch.cuda.synchronize()
    return tuple(r.cpu().numpy() for r in res)


def _ratio_of(w, b, c, cur_r):
    x = int(w.tokens[b, c])
    qx = np.float64(w.qdraft[b, c, x])
    rx = cur_r[x]
    if rx == 0:
        return 0.0
    if qx == 0:
        return np.inf
    return rx / qx


def check_sample(w, got, want):
    """Bit-exact decisions in walk order until a test falls within the band
    |u - ratio| < 1e-6 (the row is then exempt); bonus equal unless exempt or
    the inverse-CDF draw sits within 1e-6 of a boundary. Returns the number of
    exempt rows."""
    al, path, bonus, am, dec, st = got
    al_r, path_r, bonus_r, am_r, dec_r, st_r = want
    assert np.array_equal(st, st_r)
    exempt = 0
    for b in range(w.B):
        n = int(w.n_nodes[b])
        if st_r[b] != 0 or n == 0:
            assert al[b] == 0 and bonus[b] == -1 and np.all(path[b] == -1)
            continue
        # Replay the oracle's walk to know each tested ratio.
        cur = 0
        r = oracle.sample_probs(w.logits[b, 0], w.temperature)
        row_exempt = False
        while True:
            kids = [c for c in range(1, n) if w.parent[b, c] == cur]
            nxt = None
            for c in kids:
                ratio = _ratio_of(w, b, c, r)
                if abs(np.float64(w.u[b, c]) - ratio) < SAMPLE_BAND:
                    row_exempt = True
                    break
                assert dec[b, c] == dec_r[b, c], (b, c, dec[b, c], dec_r[b, c], ratio)
                if dec_r[b, c] == 1:
                    nxt = c
                    break
                qc = w.qdraft[b, c].astype(np.float64)
                res = np.maximum(r - qc, 0.0)
                if res.sum() > 0:
                    r = res / res.sum()
            if row_exempt or nxt is None:
                break
            cur = nxt
            r = oracle.sample_probs(w.logits[b, cur], w.temperature)
        if row_exempt:
            exempt += 1
            continue
        assert al[b] == al_r[b] and np.array_equal(path[b], path_r[b])
        assert np.array_equal(am[b], am_r[b]) and np.array_equal(dec[b], dec_r[b])
        if bonus[b] != bonus_r[b]:
            c = np.cumsum(r)
            thr = np.float64(w.u[b, 0]) * c[-1]
            lo, hi = sorted((int(bonus[b]), int(bonus_r[b])))
            near = np.min(np.abs(c[lo:hi + 1] - thr))
            assert near < SAMPLE_BAND * c[-1], (b, bonus[b], bonus_r[b])
            exempt += 1
    return exempt
