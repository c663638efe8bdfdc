"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/tv.h declares, and rejects bad arguments with the
documented status codes before any HIP call."""

import ctypes
import os
import re

import pytest

import tree_attention_draft_tv_amd as tv
from tree_attention_draft_tv_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tv.h")

# Non-null, 256-byte aligned fake addresses: validation must fail before use.
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
NULL = None
STREAM = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tv.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(binding.SIGNATURES) == names


def test_version_and_status_strings(lib):
    assert lib.tv_version() == 100
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 1, 2, 3, 4, 5, 6):
        s = lib.tv_status_string(code).decode()
        assert s and s != "unknown status", code
    assert lib.tv_status_string(99).decode() == "unknown status"


def test_mask_validation(lib):
    assert lib.tv_build_tree_mask(NULL, P, 1, 4, P, P, P, STREAM) == -1
    assert lib.tv_build_tree_mask(P, P, 1, 0, P, P, P, STREAM) == -2
    assert lib.tv_build_tree_mask(P, P, 1, 129, P, P, P, STREAM) == -2
    assert lib.tv_build_tree_mask(P, P, -1, 4, P, P, P, STREAM) == -2
    assert lib.tv_build_tree_mask(P, P, 0, 4, P, P, P, STREAM) == 0  # nothing to do


def test_block_mask_validation(lib):
    assert lib.tv_build_block_mask(NULL, 1, 4, 0, P, P, P, STREAM) == -1
    assert lib.tv_build_block_mask(P, 1, 4, 0, NULL, P, P, STREAM) == -1
    assert lib.tv_build_block_mask(P, 1, 0, 0, P, P, P, STREAM) == -2
    assert lib.tv_build_block_mask(P, 1, 129, 1, P, P, P, STREAM) == -2
    assert lib.tv_build_block_mask(P, -1, 4, 0, P, P, P, STREAM) == -2
    assert lib.tv_build_block_mask(P, 1, 4, 2, P, P, P, STREAM) == -6
    assert lib.tv_build_block_mask(P, 0, 4, 1, P, P, P, STREAM) == 0


def _attn(lib, **kw):
    a = dict(q=P, q_sb=8 * 33 * 28 * 128, q_st=28 * 128, q_sh=128, k=P, v=P2,
             kv_sb=4 * 4096 * 128, kv_sh=4096 * 128, kv_ss=128, ctx=P, n=P, mask=P,
             B=2, T=33, Hq=28, Hkv=4, D=128, max_ctx=4000, cap=4096, scale=0.088,
             dtype=1, out_dtype=0, parts=3, chunk=0, out=P, lse=P, ws=P, ws_bytes=1 << 40, st=P)
    a.update(kw)
    return lib.tv_tree_attention(a["q"], a["q_sb"], a["q_st"], a["q_sh"], a["k"], a["v"],
                                 a["kv_sb"], a["kv_sh"], a["kv_ss"], a["ctx"], a["n"], a["mask"],
                                 a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["max_ctx"],
                                 a["cap"], a["scale"], a["dtype"], a["out_dtype"], a["parts"],
                                 a["chunk"], a["out"], a["lse"], a["ws"], a["ws_bytes"], a["st"],
                                 STREAM)


def test_attention_validation(lib):
    assert _attn(lib, q=NULL) == -1
    assert _attn(lib, mask=NULL) == -1
    assert _attn(lib, st=NULL) == -1
    assert _attn(lib, dtype=5) == -3
    assert _attn(lib, out_dtype=2) == -3 and _attn(lib, out_dtype=-1) == -3
    assert _attn(lib, T=0) == -2
    assert _attn(lib, T=129) == -2
    assert _attn(lib, Hq=27) == -2                  # not a multiple of Hkv
    assert _attn(lib, Hq=68) == -2                  # group of 17 > 16
    assert _attn(lib, parts=4) == -2
    assert _attn(lib, chunk=100) == -2              # not a multiple of 64
    assert _attn(lib, chunk=32) == -2
    assert _attn(lib, cap=0) == -2
    assert _attn(lib, D=96) == -6
    assert _attn(lib, q=ctypes.c_void_p(0x100008)) == -4
    assert _attn(lib, kv_ss=132) == -4               # bf16 stride not a multiple of 8
    assert _attn(lib, ws=NULL, ws_bytes=0) == -5
    assert _attn(lib, ws_bytes=16) == -5
    assert _attn(lib, ws=ctypes.c_void_p(0x100010)) == -5  # not 256-byte aligned
    assert _attn(lib, B=0) == 0


def _attn_packed(lib, **kw):
    a = dict(q=P, q_st=28 * 128, q_sh=128, k=P, v=P2, kv_sb=4 * 4096 * 128, kv_sh=4096 * 128,
             kv_ss=128, ctx=P, n=P, mask=P, start=P, rows=100, B=2, T=33, Hq=28, Hkv=4, D=128,
             max_ctx=4000, cap=4096, scale=0.088, dtype=1, out_dtype=1, parts=3, chunk=0, out=P,
             lse=P, ws=P, ws_bytes=1 << 40, st=P)
    a.update(kw)
    return lib.tv_tree_attention_packed(
        a["q"], a["q_st"], a["q_sh"], a["k"], a["v"], a["kv_sb"], a["kv_sh"], a["kv_ss"],
        a["ctx"], a["n"], a["mask"], a["start"], a["rows"], a["B"], a["T"], a["Hq"], a["Hkv"],
        a["D"], a["max_ctx"], a["cap"], a["scale"], a["dtype"], a["out_dtype"], a["parts"],
        a["chunk"], a["out"], a["lse"], a["ws"], a["ws_bytes"], a["st"], STREAM)


def test_attention_packed_validation(lib):
    assert _attn_packed(lib, start=NULL) == -1
    assert _attn_packed(lib, q=NULL) == -1
    assert _attn_packed(lib, rows=-1) == -2
    assert _attn_packed(lib, T=129) == -2
    assert _attn_packed(lib, dtype=7) == -3
    assert _attn_packed(lib, out_dtype=3) == -3
    assert _attn_packed(lib, q_st=28 * 128 + 4) == -4   # row stride not 16 bytes
    assert _attn_packed(lib, D=80) == -6
    assert _attn_packed(lib, ws=NULL, ws_bytes=0) == -5
    assert _attn_packed(lib, B=0) == 0
    assert _attn_packed(lib, B=0, rows=0) == 0


def _budget(lib, **kw):
    a = dict(acc=P, n=P, st=NULL, B=4, target=0.5, alpha=0.25, n_min=1, n_max=64, ema=P,
             budget=P, start=P, total=P)
    a.update(kw)
    return lib.tv_adapt_tree_budget(a["acc"], a["n"], a["st"], a["B"], a["target"], a["alpha"],
                                    a["n_min"], a["n_max"], a["ema"], a["budget"], a["start"],
                                    a["total"], STREAM)


def test_budget_validation(lib):
    assert _budget(lib, acc=NULL) == -1
    assert _budget(lib, ema=NULL) == -1
    assert _budget(lib, total=NULL) == -1
    assert _budget(lib, B=0, total=NULL) == -1
    assert _budget(lib, B=-1) == -2
    assert _budget(lib, target=1.5) == -2 and _budget(lib, target=-0.1) == -2
    assert _budget(lib, target=float("nan")) == -2
    assert _budget(lib, alpha=0.0) == -2 and _budget(lib, alpha=1.01) == -2
    assert _budget(lib, n_min=0) == -2
    assert _budget(lib, n_min=5, n_max=4) == -2
    assert _budget(lib, n_max=128) == -2                 # at most TV_MAX_TREE - 1 draft nodes
    assert _budget(lib, B=1 << 24) == -2                 # row table would overflow int32


def test_attention_workspace_size(lib):
    f = lib.tv_tree_attention_workspace_size
    assert f(8, 33, 28, 4, 128, 256, 256) == 0          # one chunk: no workspace
    assert f(1, 9, 8, 2, 64, 0, 0) == 0               # every pair one unit: no workspace
    assert f(1, 9, 8, 2, 64, 128, 0) > 0              # balanced units may split a pair
    big = f(8, 33, 28, 4, 128, 7650, 512)
    rows = 8 * 4 * 15 * 231
    assert big >= rows * (128 * 4 + 8)
    assert f(8, 33, 28, 4, 128, 7650, 100) == ctypes.c_size_t(-1).value
    assert lib.tv_tree_attention_auto_chunk(8, 33, 28, 4, 7650) % 64 == 0


def test_accept_validation(lib):
    g = lib.tv_accept_greedy
    ok = dict(lg=P, stride=152064, tok=P, par=P, n=P, B=2, T=33, V=152064, al=P, path=P,
              bonus=P, am=P, ws=P, wsb=1 << 40, st=P)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["lg"], a["stride"], a["tok"], a["par"], a["n"], a["B"], a["T"], a["V"],
                 a["al"], a["path"], a["bonus"], a["am"], a["ws"], a["wsb"], a["st"], STREAM)

    assert call(lg=NULL) == -1
    assert call(bonus=NULL) == -1
    assert call(T=0) == -2 and call(T=200) == -2 and call(V=0) == -2
    assert call(stride=100) == -2
    assert call(lg=ctypes.c_void_p(0x100002)) == -4      # not even float-aligned
    assert call(ws=NULL) == -5 and call(wsb=8) == -5
    assert call(B=0) == 0
    s = lib.tv_accept_sample

    def scall(**kw):
        a = dict(lg=P, stride=32000, temp=0.7, q=P2, qs=32000, u=P, tok=P, par=P, n=P, B=2,
                 T=33, V=32000, al=P, path=P, bonus=P, am=P, dec=P, ws=P, wsb=1 << 40, st=P)
        a.update(kw)
        return s(a["lg"], a["stride"], a["temp"], a["q"], a["qs"], a["u"], a["tok"], a["par"],
                 a["n"], a["B"], a["T"], a["V"], a["al"], a["path"], a["bonus"], a["am"],
                 a["dec"], a["ws"], a["wsb"], a["st"], STREAM)

    assert scall(q=NULL) == -1 and scall(dec=NULL) == -1 and scall(u=NULL) == -1
    assert scall(temp=0.0) == -2 and scall(temp=-1.0) == -2
    assert scall(qs=10) == -2
    assert scall(q=ctypes.c_void_p(0x200001)) == -4
    assert scall(wsb=100) == -5
    assert scall(B=65536) == -2
    assert scall(B=0) == 0


def test_accept_workspace_size(lib):
    f = lib.tv_accept_workspace_size
    assert f(8, 33, 152064, 0) >= 8 * 33 * 10 * 8
    # Sampling up to V = 32768: per node an accepted child, a bonus and a
    # decision byte; larger vocabularies keep float64 rows.
    assert f(8, 33, 32000, 1) >= 8 * 33 * 9
    assert f(8, 33, 32000, 1) < 8 * 32000
    assert f(8, 33, 152064, 1) >= 8 * 33 * 152064 * 8
    assert f(8, 33, 32000, 2) == ctypes.c_size_t(-1).value
    assert f(8, 0, 32000, 0) == ctypes.c_size_t(-1).value


def test_python_binding_rejects_cpu_tensors():
    import torch
    parent = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(tv.TVError, match="GPU"):
        tv.build_tree_mask(parent, torch.ones(1, dtype=torch.int32))


def test_python_binding_rejects_wrong_shapes_before_launch():
    # Shapes are checked before the device, so these raise on the host (the
    # tensors are CPU tensors: a call that got as far as a launch would
    # instead fail on the device check).
    import torch
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    B, T, Hq, Hkv, D, cap = 2, 9, 8, 2, 64, 128
    q, k, v = f32(B, T, Hq, D), f32(B, Hkv, cap, D), f32(B, Hkv, cap, D)
    mask = i32(B, T, 1)

    def attn(**kw):
        a = dict(ctx=i32(B), n=i32(B), mask=mask)
        a.update(kw)
        return tv.tree_attention(q, k, v, a.pop("ctx"), a.pop("n"), a.pop("mask"), 100, **a)

    for kw, what in ((dict(ctx=i32(B + 1)), "ctx_len"), (dict(n=i32(1)), "n_nodes"),
                     (dict(mask=i32(B, T, 2)), "mask"), (dict(out=f32(B, T, Hq, D + 1)), "out"),
                     (dict(lse=f32(B, T)), "lse"), (dict(row_status=i32(B + 1)), "row_status")):
        with pytest.raises(tv.TVError, match=what):
            attn(**kw)
    with pytest.raises(TypeError):
        attn(out=torch.zeros((B, T, Hq, D), dtype=torch.float64))
    with pytest.raises(TypeError):
        attn(out_dtype=torch.float16)
    with pytest.raises(tv.TVError, match="row_start"):
        tv.tree_attention_packed(f32(20, Hq, D), k, v, i32(B), i32(B), mask, i32(B + 2), 100)
    logits = f32(B, T, 50)
    outs = (i32(B), i32(B, T), i32(B), torch.zeros((B, T), dtype=torch.uint8), i32(B))
    with pytest.raises(tv.TVError, match="n_nodes"):
        tv.accept_greedy(logits, i32(B, T), i32(B, T), i32(B + 1))
    bad = (i32(B + 1),) + outs[1:]
    with pytest.raises(tv.TVError, match="accept_len"):
        tv.accept_greedy(logits, i32(B, T), i32(B, T), i32(B), outputs=bad)
    bad = outs[:3] + (torch.zeros((B, T + 1), dtype=torch.uint8), outs[4])
    with pytest.raises(tv.TVError, match="accept_mask"):
        tv.accept_greedy(logits, i32(B, T), i32(B, T), i32(B), outputs=bad)
    dec = torch.zeros((B, T), dtype=torch.int8)
    with pytest.raises(tv.TVError, match="decision"):
        tv.accept_sample(logits, 0.7, f32(B, T, 50), f32(B, T), i32(B, T), i32(B, T), i32(B),
                         outputs=outs[:4] + (dec[:1], outs[4]))
    with pytest.raises(tv.TVError, match="u"):
        tv.accept_sample(logits, 0.7, f32(B, T, 50), f32(B, T + 1), i32(B, T), i32(B, T), i32(B))
    with pytest.raises(tv.TVError, match="mask"):
        tv.build_tree_mask(i32(B, T), i32(B), out=(i32(B, T, 2), i32(B, T), i32(B)))
    with pytest.raises(tv.TVError, match="accept_len"):
        tv.commit_accepted_kv(k, v, i32(B), i32(B), i32(B + 1), i32(B, T))


def _commit(lib, **kw):
    a = dict(k=P, v=P2, layer_stride=0, kv_sb=4 * 8192 * 128, kv_sh=8192 * 128, kv_ss=128,
             ctx=P, n=P, acc=P, path=P, B=8, T=33, Hkv=4, D=128, elem=2, layers=1, cap=8192,
             new_ctx=P2, st=P2)
    a.update(kw)
    return lib.tv_commit_accepted_kv(a["k"], a["v"], a["layer_stride"], a["kv_sb"], a["kv_sh"],
                                     a["kv_ss"], a["ctx"], a["n"], a["acc"], a["path"], a["B"],
                                     a["T"], a["Hkv"], a["D"], a["elem"], a["layers"], a["cap"],
                                     a["new_ctx"], a["st"], STREAM)


def test_commit_validation(lib):
    assert _commit(lib, k=NULL) == -1
    assert _commit(lib, path=NULL) == -1
    assert _commit(lib, elem=8) == -3
    assert _commit(lib, T=0) == -2
    assert _commit(lib, T=129) == -2
    assert _commit(lib, layers=0) == -2
    assert _commit(lib, B=-1) == -2
    assert _commit(lib, D=4) == -6          # 8-byte rows
    assert _commit(lib, D=512) == -6        # 1024-byte rows
    assert _commit(lib, kv_ss=129) == -4    # stride not a multiple of 16 bytes
    assert _commit(lib, k=ctypes.c_void_p(0x100008)) == -4
    assert _commit(lib, new_ctx=P) == -2    # new_ctx_len may not be ctx_len
    assert _commit(lib, B=0) == 0           # nothing to do


def test_linear_validation(lib):
    f = lib.tv_linear_rows
    assert f(NULL, 3584, P, 3584, 264, 3584, 4608, P2, 4608, STREAM) == -1
    assert f(P, 3584, P, 3584, 264, 3584 + 32, 4608, P2, 4608, STREAM) == -2   # K % 64
    assert f(P, 3584, P, 3584, 264, 3584, 4608 + 32, P2, 4608 + 32, STREAM) == -2  # N % 64
    assert f(P, 3584, P, 3584, -1, 3584, 4608, P2, 4608, STREAM) == -2
    assert f(P, 3580, P, 3584, 264, 3584, 4608, P2, 4608, STREAM) == -2     # x_stride < K
    assert f(P, 3592 + 4, P, 3584, 264, 3584, 4608, P2, 4608, STREAM) == -4  # x_stride % 8
    assert f(ctypes.c_void_p(0x100008), 3584, P, 3584, 264, 3584, 4608, P2, 4608, STREAM) == -4
    assert f(P, 3584, P, 3584, 0, 3584, 4608, P2, 4608, STREAM) == 0
    g = lib.tv_linear_swiglu_rows
    assert g(P, 3584, P, NULL, 3584, 264, 3584, 18944, P2, 18944, STREAM) == -1
    assert g(P, 3584, P, P, 3584, 0, 3584, 18944, P2, 18944, STREAM) == 0


def test_accept_greedy_noalloc_validation(lib):
    f = lib.tv_accept_greedy_noalloc

    def call(**kw):
        a = dict(lg=P, stride=152064, tok=P, par=P, n=P, B=8, T=33, V=152064, al=P, path=P,
                 bonus=P, am=P, st=P)
        a.update(kw)
        return f(a["lg"], a["stride"], a["tok"], a["par"], a["n"], a["B"], a["T"], a["V"],
                 a["al"], a["path"], a["bonus"], a["am"], a["st"], STREAM)

    assert call(lg=NULL) == -1 and call(st=NULL) == -1
    assert call(T=0) == -2 and call(V=0) == -2 and call(stride=10) == -2
    assert call(B=65536) == -2
    assert call(lg=ctypes.c_void_p(0x100002)) == -4
    assert call(B=0) == 0
    # Beyond the 2 MiB static scratch: B * T * slices * 8 bytes. Rejected on
    # the host before the device is touched.
    big = lib.tv_accept_workspace_size(1024, 33, 152064, 0)
    assert big > (2 << 20)
    assert call(B=1024) == -5
    assert lib.tv_accept_workspace_size(512, 33, 152064, 0) <= (2 << 20)


def test_read_probe_validation(lib):
    f = lib.tv_read_probe
    P = ctypes.c_void_p(0x100000)
    assert f(None, 1024, P, STREAM) == -1
    assert f(P, 1024, None, STREAM) == -1
    assert f(P, 0, P, STREAM) == -2
    assert f(P, 1000, P, STREAM) == -2
    assert f(ctypes.c_void_p(0x100004), 1024, P, STREAM) == -4
