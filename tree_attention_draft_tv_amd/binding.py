"""Thin Python binding of the tree-verification C ABI (``include/tv.h``).

Argument marshalling only: every step runs in the HIP kernels of
``libtv.so``. PyTorch provides device memory and the current HIP stream;
the functions take and return torch tensors on an MI355X device. There is
no fallback: if ``libtv.so`` is missing or a call fails, an exception is
raised.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtv.so")

TV_F32 = 0
TV_BF16 = 1
TV_BLOCK_CAUSAL = 0
TV_BLOCK_BIDIRECTIONAL = 1
TV_MAX_TREE = 128
TV_MAX_GROUP = 16

STATUS = {
    0: "TV_OK", -1: "TV_ERR_NULL", -2: "TV_ERR_SHAPE", -3: "TV_ERR_DTYPE",
    -4: "TV_ERR_ALIGN", -5: "TV_ERR_WORKSPACE", -6: "TV_ERR_UNSUPPORTED", -7: "TV_ERR_HIP",
}
ROW_STATUS = {0: "TV_ROW_OK", 1: "TV_ROW_BAD_PARENT", 2: "TV_ROW_CTX_BOUND",
              3: "TV_ROW_NNODES", 4: "TV_ROW_BAD_TOKEN", 5: "TV_ROW_BAD_PATH",
              6: "TV_ROW_BAD_START"}

# Every exported symbol of include/tv.h with its (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_S = ctypes.c_size_t
_F = ctypes.c_float
SIGNATURES = {
    "tv_build_tree_mask": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "tv_build_block_mask": (_I, [_P, _I, _I, _I, _P, _P, _P, _P]),
    "tv_tree_attention_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "tv_tree_attention_auto_chunk": (_I, [_I, _I, _I, _I, _I]),
    "tv_tree_attention": (_I, [_P, _L, _L, _L, _P, _P, _L, _L, _L, _P, _P, _P,
                               _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                               _P, _P, _P, _S, _P, _P]),
    "tv_tree_attention_packed": (_I, [_P, _L, _L, _P, _P, _L, _L, _L, _P, _P, _P, _P, _I,
                                      _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I,
                                      _P, _P, _P, _S, _P, _P]),
    "tv_adapt_tree_budget": (_I, [_P, _P, _P, _I, _F, _F, _I, _I, _P, _P, _P, _P, _P]),
    "tv_accept_workspace_size": (_S, [_I, _I, _I, _I]),
    "tv_accept_greedy": (_I, [_P, _L, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _S, _P, _P]),
    "tv_accept_greedy_noalloc": (_I, [_P, _L, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "tv_accept_sample": (_I, [_P, _L, _F, _P, _L, _P, _P, _P, _P, _I, _I, _I,
                              _P, _P, _P, _P, _P, _P, _S, _P, _P]),
    "tv_commit_accepted_kv": (_I, [_P, _P, _L, _L, _L, _L, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                   _I, _P, _P, _P]),
    "tv_linear_rows": (_I, [_P, _L, _P, _L, _I, _I, _I, _P, _L, _P]),
    "tv_linear_swiglu_rows": (_I, [_P, _L, _P, _P, _L, _I, _I, _I, _P, _L, _P]),
    "tv_read_probe": (_I, [_P, _S, _P, _P]),
    "tv_status_string": (ctypes.c_char_p, [_I]),
    "tv_version": (_I, []),
}

_lib = None


class TVError(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libtv.so`` once and declare every signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise TVError("libtv.so is not built (%s); run __graft_entry__.build() or "
                      "python -m tree_attention_draft_tv_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, what: str):
    if code != 0:
        msg = load().tv_status_string(code).decode()
        raise TVError("%s failed: %s (%s)" % (what, STATUS.get(code, code), msg))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(t: torch.Tensor, name: str, dtype, shape=None, contiguous=False):
    """Type, element type, shape and layout of an argument (no device check)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise TVError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if contiguous and not t.is_contiguous():
        raise TVError("%s must be contiguous" % name)


def _need(t: torch.Tensor, name: str, dtype, device=None, shape=None, contiguous=False):
    """:func:`_shape`, then the device."""
    _shape(t, name, dtype, shape, contiguous)
    if t.device.type != "cuda":
        raise TVError("%s must live on the GPU (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise TVError("%s is on %s, expected %s" % (name, t.device, device))


def _out_dtype(dtype):
    if dtype == torch.float32:
        return TV_F32
    if dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
            raise TVError("workspace must be a contiguous tensor")
        if workspace.device != device:
            raise TVError("workspace is on %s, expected %s" % (workspace.device, device))
        if workspace.numel() * workspace.element_size() < nbytes:
            raise TVError("workspace too small: %d < %d bytes" %
                          (workspace.numel() * workspace.element_size(), nbytes))
        return workspace, workspace.numel() * workspace.element_size()
    # The caching allocator returns 256-byte aligned blocks.
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ----------------------------------------------------------------- mask ---

def build_tree_mask(parent: torch.Tensor, n_nodes: torch.Tensor,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Ancestor bitmasks (int32 storage of uint32 words), depths, row status."""
    lib = load()
    dev = parent.device
    if not isinstance(parent, torch.Tensor) or parent.dim() != 2:
        raise TVError("parent must be a contiguous [B, T] tensor")
    B, T = parent.shape
    W = (T + 31) // 32
    checks = [(parent, "parent", (B, T)), (n_nodes, "n_nodes", (B,))]
    if out is not None:
        checks += list(zip(out, ("mask", "depth", "row_status"), ((B, T, W), (B, T), (B,))))
    for t, name, shape in checks:
        _shape(t, name, torch.int32, shape, contiguous=True)
    for t, name, _ in checks:
        _need(t, name, torch.int32, dev)
    if out is None:
        mask = torch.empty((B, T, W), dtype=torch.int32, device=dev)
        depth = torch.empty((B, T), dtype=torch.int32, device=dev)
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        mask, depth, status = out
    _check(lib.tv_build_tree_mask(_ptr(parent), _ptr(n_nodes), B, T, _ptr(mask), _ptr(depth),
                                  _ptr(status), _stream(dev)), "tv_build_tree_mask")
    return mask, depth, status


def build_block_mask(n_nodes: torch.Tensor, T: int, mode: int = TV_BLOCK_CAUSAL,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Masks of a draft block (TV_BLOCK_CAUSAL or TV_BLOCK_BIDIRECTIONAL) in
    the layout of :func:`build_tree_mask`: (mask, position, row_status)."""
    lib = load()
    dev = n_nodes.device
    if not isinstance(n_nodes, torch.Tensor) or n_nodes.dim() != 1:
        raise TVError("n_nodes must be a contiguous [B] tensor")
    B = n_nodes.shape[0]
    T = int(T)
    W = (T + 31) // 32
    checks = [(n_nodes, "n_nodes", (B,))]
    if out is not None:
        checks += list(zip(out, ("mask", "position", "row_status"), ((B, T, W), (B, T), (B,))))
    for t, name, shape in checks:
        _shape(t, name, torch.int32, shape, contiguous=True)
    for t, name, _ in checks:
        _need(t, name, torch.int32, dev)
    if out is None:
        mask = torch.empty((B, T, W), dtype=torch.int32, device=dev)
        pos = torch.empty((B, T), dtype=torch.int32, device=dev)
        status = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        mask, pos, status = out
    _check(lib.tv_build_block_mask(_ptr(n_nodes), B, int(T), int(mode), _ptr(mask), _ptr(pos),
                                   _ptr(status), _stream(dev)), "tv_build_block_mask")
    return mask, pos, status


# ------------------------------------------------------------ attention ---

def attention_workspace_size(B, T, Hq, Hkv, D, max_ctx, chunk_keys=0) -> int:
    n = load().tv_tree_attention_workspace_size(B, T, Hq, Hkv, D, max_ctx, chunk_keys)
    if n == ctypes.c_size_t(-1).value:
        raise TVError("invalid attention sizes")
    return int(n)


def auto_chunk(B, T, Hq, Hkv, max_ctx) -> int:
    return int(load().tv_tree_attention_auto_chunk(B, T, Hq, Hkv, max_ctx))


def _attention_args(q, k, v, ctx_len, n_nodes, mask, B, T, lead, Hq, D, out_dtype, out, lse,
                    row_status):
    """Checks every attention argument (all shapes before any device) and
    allocates the outputs not given: out [*lead, Hq, D] of out_dtype, lse
    float32 [*lead, Hq], row_status int32 [B]. Returns (element type code,
    out, lse, row_status)."""
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch tensor")
    if q.dtype == torch.bfloat16:
        dt = TV_BF16
    elif q.dtype == torch.float32:
        dt = TV_F32
    else:
        raise TypeError("q must be float32 or bfloat16")
    _out_dtype(out_dtype)
    o_shape, l_shape = tuple(lead) + (Hq, D), tuple(lead) + (Hq,)
    checks = [(ctx_len, "ctx_len", torch.int32, (B,)), (n_nodes, "n_nodes", torch.int32, (B,)),
              (mask, "mask", torch.int32, (B, T, (T + 31) // 32)),
              (out, "out", out_dtype, o_shape), (lse, "lse", torch.float32, l_shape),
              (row_status, "row_status", torch.int32, (B,))]
    _shape(k, "k", q.dtype)
    _shape(v, "v", q.dtype)
    for t, name, dtype, shape in checks:
        if t is not None:
            _shape(t, name, dtype, shape, contiguous=True)
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, q.dtype, dev)
    for t, name, dtype, _ in checks:
        if t is not None:
            _need(t, name, dtype, dev)
    if out is None:
        out = torch.empty(o_shape, dtype=out_dtype, device=dev)
    if lse is None:
        lse = torch.empty(l_shape, dtype=torch.float32, device=dev)
    if row_status is None:
        row_status = torch.empty((B,), dtype=torch.int32, device=dev)
    return dt, out, lse, row_status


def tree_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, ctx_len: torch.Tensor,
                   n_nodes: torch.Tensor, mask: torch.Tensor, max_ctx: int,
                   scale: Optional[float] = None, probability_parts: int = 3,
                   chunk_keys: int = 0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, row_status: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32):
    """Tree-masked split-KV GQA attention.

    q: [B, T, Hq, D]; k, v: [B, Hkv, kv_capacity, D] (float32 or bfloat16,
    D contiguous, any other strides); ctx_len, n_nodes: int32 [B];
    mask: from :func:`build_tree_mask`. ``probability_parts`` 3 (default)
    keeps the probabilities fp32-faithful; 1 is the lossy fast mode described
    in include/tv.h. Returns (out [B, T, Hq, D] of ``out_dtype`` (float32 or
    bfloat16), lse float32 [B, T, Hq], row_status int32 [B]).
    """
    lib = load()
    if not isinstance(q, torch.Tensor) or q.dim() != 4 or not isinstance(k, torch.Tensor) or \
            k.dim() != 4 or not isinstance(v, torch.Tensor) or v.shape != k.shape:
        raise TVError("q must be [B, T, Hq, D] and k, v [B, Hkv, capacity, D]")
    B, T, Hq, D = q.shape
    _, Hkv, cap, Dk = k.shape
    if Dk != D or k.shape[0] != B:
        raise TVError("q and k disagree on B or D")
    dt, out, lse, row_status = _attention_args(q, k, v, ctx_len, n_nodes, mask, B, T, (B, T),
                                               Hq, D, out_dtype, out, lse, row_status)
    dev = q.device
    if q.stride(3) != 1 or k.stride(3) != 1 or v.stride(3) != 1:
        raise TVError("the head dimension must be contiguous")
    if k.stride() != v.stride():
        raise TVError("k and v must share strides")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    odt = _out_dtype(out_dtype)
    nbytes = attention_workspace_size(B, T, Hq, Hkv, D, max_ctx, chunk_keys)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    _check(lib.tv_tree_attention(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2),
        _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(ctx_len), _ptr(n_nodes), _ptr(mask),
        B, T, Hq, Hkv, D, int(max_ctx), cap, float(scale), dt, odt, int(probability_parts),
        int(chunk_keys), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _ptr(row_status),
        _stream(dev)), "tv_tree_attention")
    return out, lse, row_status


def tree_attention_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          ctx_len: torch.Tensor, n_nodes: torch.Tensor, mask: torch.Tensor,
                          row_start: torch.Tensor, max_ctx: int, scale: Optional[float] = None,
                          probability_parts: int = 3, chunk_keys: int = 0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          row_status: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          out_dtype: torch.dtype = torch.float32):
    """:func:`tree_attention` over packed query rows: node i of sequence b is
    row row_start[b] + i of q [rows, Hq, D], out [rows, Hq, D] and lse
    [rows, Hq]; the query extent T (largest n_nodes accepted) is the mask's
    second dimension (mask: [B, T, ceil(T/32)], as for the padded call).
    Rows of no live sequence are left as they are (``out``/``lse`` given) or
    uninitialised. Returns (out, lse, row_status)."""
    lib = load()
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not isinstance(k, torch.Tensor) or \
            k.dim() != 4 or not isinstance(v, torch.Tensor) or v.shape != k.shape:
        raise TVError("q must be [rows, Hq, D] and k, v [B, Hkv, capacity, D]")
    rows, Hq, D = q.shape
    B, Hkv, cap, Dk = k.shape
    if Dk != D:
        raise TVError("q and k disagree on D")
    if not isinstance(mask, torch.Tensor) or mask.dim() != 3:
        raise TVError("mask must be a contiguous [B, T, ceil(T/32)] tensor")
    T = mask.shape[1]
    _shape(row_start, "row_start", torch.int32, shape=(B,), contiguous=True)
    dt, out, lse, row_status = _attention_args(q, k, v, ctx_len, n_nodes, mask, B, T, (rows,),
                                               Hq, D, out_dtype, out, lse, row_status)
    dev = q.device
    _need(row_start, "row_start", torch.int32, dev)
    if q.stride(2) != 1 or k.stride(3) != 1 or v.stride(3) != 1:
        raise TVError("the head dimension must be contiguous")
    if k.stride() != v.stride():
        raise TVError("k and v must share strides")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    odt = _out_dtype(out_dtype)
    nbytes = attention_workspace_size(B, T, Hq, Hkv, D, max_ctx, chunk_keys)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    _check(lib.tv_tree_attention_packed(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), _ptr(v), k.stride(0), k.stride(1),
        k.stride(2), _ptr(ctx_len), _ptr(n_nodes), _ptr(mask), _ptr(row_start), rows,
        B, T, Hq, Hkv, D, int(max_ctx), cap, float(scale), dt, odt, int(probability_parts),
        int(chunk_keys), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _ptr(row_status),
        _stream(dev)), "tv_tree_attention_packed")
    return out, lse, row_status


def adapt_tree_budget(accept_len: torch.Tensor, n_nodes: torch.Tensor,
                      ratio_ema: torch.Tensor, budget: torch.Tensor, target: float,
                      alpha: float, n_min: int, n_max: int,
                      row_status: Optional[torch.Tensor] = None,
                      row_start: Optional[torch.Tensor] = None,
                      rows_total: Optional[torch.Tensor] = None):
    """Device-side adaptive draft budget: updates ``ratio_ema`` (float32 [B])
    and ``budget`` (int32 [B]) in place from the last step's acceptance and
    returns (row_start int32 [B], rows_total int32 [1]), the packed row table
    of the next step (budget + 1 rows per sequence)."""
    lib = load()
    dev = accept_len.device
    _need(accept_len, "accept_len", torch.int32)
    _need(n_nodes, "n_nodes", torch.int32, dev)
    _need(ratio_ema, "ratio_ema", torch.float32, dev)
    _need(budget, "budget", torch.int32, dev)
    B = accept_len.shape[0]
    for t, name in ((accept_len, "accept_len"), (n_nodes, "n_nodes"), (ratio_ema, "ratio_ema"),
                    (budget, "budget")):
        if tuple(t.shape) != (B,) or not t.is_contiguous():
            raise TVError(name + " must be a contiguous [B] tensor")
    if row_status is not None:
        _need(row_status, "row_status", torch.int32, dev)
        if tuple(row_status.shape) != (B,):
            raise TVError("row_status must be [B]")
    if row_start is None:
        row_start = torch.empty((B,), dtype=torch.int32, device=dev)
    if rows_total is None:
        rows_total = torch.empty((1,), dtype=torch.int32, device=dev)
    _need(row_start, "row_start", torch.int32, dev, shape=(B,), contiguous=True)
    _need(rows_total, "rows_total", torch.int32, dev, shape=(1,), contiguous=True)
    _check(lib.tv_adapt_tree_budget(
        _ptr(accept_len), _ptr(n_nodes), _ptr(row_status), B, float(target), float(alpha),
        int(n_min), int(n_max), _ptr(ratio_ema), _ptr(budget), _ptr(row_start),
        _ptr(rows_total), _stream(dev)), "tv_adapt_tree_budget")
    return row_start, rows_total


# ----------------------------------------------------------- acceptance ---

def accept_workspace_size(B, T, V, mode) -> int:
    n = load().tv_accept_workspace_size(B, T, V, mode)
    if n == ctypes.c_size_t(-1).value:
        raise TVError("invalid acceptance sizes")
    return int(n)


def _accept_outputs(B, T, dev):
    return (torch.empty((B,), dtype=torch.int32, device=dev),
            torch.empty((B, T), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev),
            torch.empty((B, T), dtype=torch.uint8, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev))


_ACCEPT_OUT = (("accept_len", torch.int32, 1), ("path", torch.int32, 2),
               ("bonus", torch.int32, 1), ("accept_mask", torch.uint8, 2),
               ("row_status", torch.int32, 1))


def _check_accept_outputs(outs, B, T, dev, with_decision=False):
    """Shapes and types of caller-given acceptance outputs; with dev, also
    their device."""
    spec = list(_ACCEPT_OUT)
    if with_decision:
        spec.insert(4, ("decision", torch.int8, 2))
    if len(outs) != len(spec):
        raise TVError("outputs must hold %d tensors" % len(spec))
    for t, (name, dtype, nd) in zip(outs, spec):
        _shape(t, name, dtype, shape=(B,) if nd == 1 else (B, T), contiguous=True)
        if dev is not None:
            _need(t, name, dtype, dev)


def _check_logits(logits, name, dev):
    _need(logits, name, torch.float32, dev)
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(0) != logits.shape[1] * logits.stride(1):
        raise TVError("%s must be [B, T, V] with V contiguous and rows evenly strided" % name)
    return logits.stride(1)


def accept_greedy(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                  n_nodes: torch.Tensor, outputs=None, workspace: Optional[torch.Tensor] = None):
    """Greedy acceptance. Returns (accept_len, path, bonus, accept_mask, row_status)."""
    lib = load()
    dev = logits.device
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise TVError("logits must be [B, T, V]")
    B, T, V = logits.shape
    for t, nm in ((tokens, "tokens"), (parent, "parent")):
        _shape(t, nm, torch.int32, shape=(B, T), contiguous=True)
    _shape(n_nodes, "n_nodes", torch.int32, shape=(B,), contiguous=True)
    if outputs is not None:
        _check_accept_outputs(outputs, B, T, None)
    stride = _check_logits(logits, "logits", dev)
    for t, nm in ((tokens, "tokens"), (parent, "parent"), (n_nodes, "n_nodes")):
        _need(t, nm, torch.int32, dev)
    outs = outputs if outputs is not None else _accept_outputs(B, T, dev)
    _check_accept_outputs(outs, B, T, dev)
    acc_len, path, bonus, amask, status = outs
    nbytes = accept_workspace_size(B, T, V, 0)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    _check(lib.tv_accept_greedy(_ptr(logits), stride, _ptr(tokens), _ptr(parent), _ptr(n_nodes),
                                B, T, V, _ptr(acc_len), _ptr(path), _ptr(bonus), _ptr(amask),
                                _ptr(ws), ws_bytes, _ptr(status), _stream(dev)),
           "tv_accept_greedy")
    return outs


def accept_greedy_noalloc(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                          n_nodes: torch.Tensor, outputs):
    """:func:`accept_greedy` through ``tv_accept_greedy_noalloc``: the library's
    static per-device scratch replaces the workspace, so the call allocates
    nothing. ``outputs`` (accept_len, path, bonus, accept_mask, row_status)
    must be given. Calls that overlap on one device race."""
    lib = load()
    dev = logits.device
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise TVError("logits must be [B, T, V]")
    B, T, V = logits.shape
    for t, nm in ((tokens, "tokens"), (parent, "parent")):
        _shape(t, nm, torch.int32, shape=(B, T), contiguous=True)
    _shape(n_nodes, "n_nodes", torch.int32, shape=(B,), contiguous=True)
    if outputs is None:
        raise TVError("outputs must be given: this call allocates nothing")
    _check_accept_outputs(outputs, B, T, None)
    stride = _check_logits(logits, "logits", dev)
    for t, nm in ((tokens, "tokens"), (parent, "parent"), (n_nodes, "n_nodes")):
        _need(t, nm, torch.int32, dev)
    _check_accept_outputs(outputs, B, T, dev)
    acc_len, path, bonus, amask, status = outputs
    _check(lib.tv_accept_greedy_noalloc(_ptr(logits), stride, _ptr(tokens), _ptr(parent),
                                        _ptr(n_nodes), B, T, V, _ptr(acc_len), _ptr(path),
                                        _ptr(bonus), _ptr(amask), _ptr(status), _stream(dev)),
           "tv_accept_greedy_noalloc")
    return outputs


def accept_sample(logits: torch.Tensor, temperature: float, q: torch.Tensor, u: torch.Tensor,
                  tokens: torch.Tensor, parent: torch.Tensor, n_nodes: torch.Tensor,
                  outputs=None, workspace: Optional[torch.Tensor] = None):
    """SpecInfer-style sampling acceptance.

    Returns (accept_len, path, bonus, accept_mask, decision, row_status).
    """
    lib = load()
    dev = logits.device
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise TVError("logits must be [B, T, V]")
    B, T, V = logits.shape
    if not isinstance(q, torch.Tensor) or tuple(q.shape) != (B, T, V):
        raise TVError("q must match logits' shape")
    _shape(u, "u", torch.float32, shape=(B, T), contiguous=True)
    for t, nm in ((tokens, "tokens"), (parent, "parent")):
        _shape(t, nm, torch.int32, shape=(B, T), contiguous=True)
    _shape(n_nodes, "n_nodes", torch.int32, shape=(B,), contiguous=True)
    if outputs is not None:
        _check_accept_outputs(outputs, B, T, None, with_decision=True)
    stride = _check_logits(logits, "logits", dev)
    qstride = _check_logits(q, "q", dev)
    for t, nm in ((u, "u"), (tokens, "tokens"), (parent, "parent"), (n_nodes, "n_nodes")):
        _need(t, nm, t.dtype, dev)
    if outputs is None:
        acc_len, path, bonus, amask, status = _accept_outputs(B, T, dev)
        decision = torch.empty((B, T), dtype=torch.int8, device=dev)
    else:
        _check_accept_outputs(outputs, B, T, dev, with_decision=True)
        acc_len, path, bonus, amask, decision, status = outputs
    nbytes = accept_workspace_size(B, T, V, 1)
    ws, ws_bytes = _workspace(nbytes, dev, workspace)
    _check(lib.tv_accept_sample(_ptr(logits), stride, float(temperature), _ptr(q), qstride,
                                _ptr(u), _ptr(tokens), _ptr(parent), _ptr(n_nodes), B, T, V,
                                _ptr(acc_len), _ptr(path), _ptr(bonus), _ptr(amask),
                                _ptr(decision), _ptr(ws), ws_bytes, _ptr(status), _stream(dev)),
           "tv_accept_sample")
    return acc_len, path, bonus, amask, decision, status


# ------------------------------------------------------------ KV commit ---

def commit_accepted_kv(k: torch.Tensor, v: torch.Tensor, ctx_len: torch.Tensor,
                       n_nodes: torch.Tensor, accept_len: torch.Tensor, path: torch.Tensor,
                       new_ctx_len: Optional[torch.Tensor] = None,
                       row_status: Optional[torch.Tensor] = None):
    """Move the accepted path's keys and values to the committed prefix, in place.

    k, v: [B, Hkv, kv_capacity, D] or [layers, B, Hkv, kv_capacity, D]
    (bfloat16, float16 or float32; D contiguous; k and v share strides);
    ctx_len, n_nodes, accept_len: int32 [B]; path: int32 [B, T] from the
    acceptance call. Returns (new_ctx_len int32 [B], row_status int32 [B]).
    """
    lib = load()
    dev = k.device
    sizes = {torch.bfloat16: 2, torch.float16: 2, torch.float32: 4}
    if not isinstance(k, torch.Tensor) or k.dtype not in sizes:
        raise TypeError("k must be bfloat16, float16 or float32")
    _shape(v, "v", k.dtype)
    if k.dim() == 4:
        layers, kk, vv = 1, k.unsqueeze(0), v.unsqueeze(0)
    elif k.dim() == 5:
        layers, kk, vv = k.shape[0], k, v
    else:
        raise TVError("k, v must be [B, Hkv, capacity, D] or [layers, B, Hkv, capacity, D]")
    if v.shape != k.shape or kk.stride() != vv.stride():
        raise TVError("k and v must have the same shape and strides")
    if kk.stride(4) != 1:
        raise TVError("the head dimension must be contiguous")
    _, B, Hkv, cap, D = kk.shape
    if not isinstance(path, torch.Tensor) or path.dim() != 2 or path.shape[0] != B:
        raise TVError("path must be a contiguous [B, T] tensor")
    T = path.shape[1]
    checks = [(ctx_len, "ctx_len", (B,)), (n_nodes, "n_nodes", (B,)),
              (accept_len, "accept_len", (B,)), (path, "path", (B, T)),
              (new_ctx_len, "new_ctx_len", (B,)), (row_status, "row_status", (B,))]
    for t, name, shape in checks:
        if t is not None:
            _shape(t, name, torch.int32, shape, contiguous=True)
    _need(k, "k", k.dtype)
    _need(v, "v", k.dtype, dev)
    for t, name, _ in checks:
        if t is not None:
            _need(t, name, torch.int32, dev)
    if new_ctx_len is None:
        new_ctx_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if row_status is None:
        row_status = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(new_ctx_len, "new_ctx_len", torch.int32, dev, shape=(B,), contiguous=True)
    _need(row_status, "row_status", torch.int32, dev, shape=(B,), contiguous=True)
    if new_ctx_len.data_ptr() == ctx_len.data_ptr():
        raise TVError("new_ctx_len must not be ctx_len itself")
    _check(lib.tv_commit_accepted_kv(
        _ptr(kk), _ptr(vv), kk.stride(0) if layers > 1 else 0, kk.stride(1), kk.stride(2),
        kk.stride(3), _ptr(ctx_len), _ptr(n_nodes), _ptr(accept_len), _ptr(path), B, T, Hkv, D,
        sizes[k.dtype], layers, cap, _ptr(new_ctx_len), _ptr(row_status), _stream(dev)),
        "tv_commit_accepted_kv")
    return new_ctx_len, row_status


# ---------------------------------------------------- few-row projections ---

def _linear_args(x, w, name):
    _need(x, "x", torch.bfloat16)
    _need(w, name, torch.bfloat16, x.device)
    if x.dim() != 2 or w.dim() != 2 or x.stride(1) != 1 or w.stride(1) != 1:
        raise TVError("x must be [M, K] and %s [N, K], rows contiguous" % name)
    if w.shape[1] != x.shape[1]:
        raise TVError("x and %s disagree on K" % name)


def linear_rows(x: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None):
    """y = x w^T (bfloat16 in and out, fp32 accumulation in sequential K
    order): x [M, K], w [N, K] -> y [M, N]."""
    lib = load()
    _linear_args(x, w, "w")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, x.device)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise TVError("out must be [M, N] with contiguous rows")
    _check(lib.tv_linear_rows(_ptr(x), x.stride(0), _ptr(w), w.stride(0), M, K, N, _ptr(out),
                              out.stride(0), _stream(x.device)), "tv_linear_rows")
    return out


def linear_swiglu_rows(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                       out: Optional[torch.Tensor] = None):
    """bf16(silu(g) * u) of the bfloat16-rounded gate and up projections."""
    lib = load()
    _linear_args(x, w_gate, "w_gate")
    _linear_args(x, w_up, "w_up")
    if w_gate.shape != w_up.shape or w_gate.stride() != w_up.stride():
        raise TVError("w_gate and w_up must have the same shape and strides")
    M, K = x.shape
    N = w_gate.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, x.device)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise TVError("out must be [M, N] with contiguous rows")
    _check(lib.tv_linear_swiglu_rows(_ptr(x), x.stride(0), _ptr(w_gate), _ptr(w_up),
                                     w_gate.stride(0), M, K, N, _ptr(out), out.stride(0),
                                     _stream(x.device)), "tv_linear_swiglu_rows")
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor):
    """Stream `buf` (a contiguous device tensor, 16-byte aligned, a multiple
    of 16 bytes) once and XOR it into sink[0] (int32 on the same device): a
    measurement of the streaming-read rate, not a verification step."""
    lib = load()
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous() or buf.device.type != "cuda":
        raise TVError("buf must be a contiguous device tensor")
    _need(sink, "sink", torch.int32, buf.device)
    if sink.numel() < 1:
        raise TVError("sink must hold at least one int32")
    _check(lib.tv_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                             _stream(buf.device)), "tv_read_probe")
