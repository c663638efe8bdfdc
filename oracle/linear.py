"""Few-row projections of the verification rows (oracle).

Test infrastructure only. The EmbodiInfer page "perf(activevln): grammar-trie
speculation and lossless throughput", commit "perf(activevln): batch-invariant
Triton GEMMs for decode projections": tree verification runs every linear
layer on a few dozen to a few hundred rows; the projections accumulate in
FP32 in sequential K order with no split-K, so a row's result depends neither
on the tiles nor on how many rows there are, and differs from the vendor GEMM
only by output rounding. Q, K and V share one launch; gate and up share one,
with the rounded SwiGLU in the epilogue, equal to the rounded SwiGLU of the
two projections.

The oracle is the definition: y = x W^T in float64 from the stored bfloat16
values, rounded once to bfloat16 (nearest, ties to even). Reading of "rounded
SwiGLU" (the page gives no formula): the gate and up projections are each
rounded to bfloat16 as separate projections would be, then
silu(g) * u = g / (1 + exp(-g)) * u is formed and rounded to bfloat16.
"""

import numpy as np

from .decode import decode


def round_bf16(x) -> np.ndarray:
    """float64 values -> the nearest bfloat16 value (ties to even), as float64.
    Two steps: to the nearest float32 first is exact enough here only when it
    cannot create a tie, so the rounding is done on the float64 bits."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    # bfloat16 keeps 7 fraction bits; float64 has 52: drop 45 with RNE.
    drop = np.uint64(45)
    half = np.uint64(1) << (drop - np.uint64(1))
    lsb = (bits >> drop) & np.uint64(1)
    rounded = ((bits + half - np.uint64(1) + lsb) >> drop) << drop
    out = rounded.view(np.float64).copy()
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def bf16_bits(x) -> np.ndarray:
    """bfloat16 storage patterns of float64 values already on the bfloat16 grid."""
    return (np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
            >> np.uint32(16)).astype(np.uint16)


def linear_rows(x, w):
    """x: bfloat16 patterns [M, K]; w: bfloat16 patterns [N, K] (output
    features by input features). Returns (exact float64 [M, N], the bfloat16
    rounding of it as float64 [M, N])."""
    xf = decode(x, "bf16")
    wf = decode(w, "bf16")
    y = xf @ wf.T
    return y, round_bf16(y)


def silu(t):
    t = np.asarray(t, dtype=np.float64)
    return t / (1.0 + np.exp(-t))


def swiglu_rows(x, w_gate, w_up):
    """Rounded SwiGLU of the two projections: (float64 value before the final
    rounding [M, N], its bfloat16 rounding [M, N], the rounded gate and up)."""
    _, g = linear_rows(x, w_gate)
    _, u = linear_rows(x, w_up)
    y = silu(g) * u
    return y, round_bf16(y), g, u
