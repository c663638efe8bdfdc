"""Pins of the few-row projection oracle (oracle/linear.py), no GPU.

* bfloat16 rounding: nearest with ties to even, checked with exact rational
  arithmetic (including constructed ties) and against torch's float32 ->
  bfloat16 conversion on float32 inputs (a single rounding there);
* the projection equals a brute-force triple loop on small shapes, and an
  identity weight returns its input;
* silu: silu(0) = 0, silu(t) - silu(-t) = t, silu(t) = t * expit(t) (SciPy);
* rounded SwiGLU: a hand-derived value and its composition from the two
  rounded projections.
"""

from fractions import Fraction

import numpy as np
import scipy.special
import torch

import oracle


def _nearest_bf16(x: float) -> float:
    """Exact: the bfloat16 neighbours of x bracket it; take the nearer, ties
    to the one with an even last fraction bit."""
    if x == 0.0:
        return 0.0
    f = Fraction(x)
    sign = -1 if f < 0 else 1
    f = abs(f)
    e = 0
    while f >= 2:
        f /= 2
        e += 1
    while f < 1:
        f *= 2
        e -= 1
    lo = Fraction(int(f * 128), 128)
    hi = lo + Fraction(1, 128)
    if f - lo < hi - f:
        r = lo
    elif hi - f < f - lo:
        r = hi
    else:
        r = lo if int(lo * 128) % 2 == 0 else hi
    return float(sign * r * Fraction(2) ** e)


def test_round_bf16_exact():
    rng = np.random.default_rng(0)
    x = rng.normal(size=3000) * 10.0 ** rng.integers(-20, 20, size=3000)
    # Constructed ties: midpoints of neighbouring bfloat16 values.
    base = oracle.round_bf16(rng.normal(size=200))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(base))) - 7)
    ties = base + np.sign(base) * ulp / 2
    x = np.concatenate([x, ties, [1.0, -1.0, 3.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]])
    got = oracle.round_bf16(x)
    for a, b in zip(x, got):
        assert b == _nearest_bf16(float(a)), a
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_round_bf16_matches_torch_on_float32():
    x = np.random.default_rng(1).normal(size=20000).astype(np.float32) * np.float32(37.0)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), t)


def _bf16_patterns(a):
    return oracle.linear.bf16_bits(oracle.round_bf16(a))


def test_linear_brute_force_and_identity():
    rng = np.random.default_rng(2)
    for M, K, N in ((1, 1, 1), (3, 5, 4), (7, 32, 9)):
        x = _bf16_patterns(rng.normal(size=(M, K)))
        w = _bf16_patterns(rng.normal(size=(N, K)))
        y, yr = oracle.linear_rows(x, w)
        xf, wf = oracle.decode(x, "bf16"), oracle.decode(w, "bf16")
        for m in range(M):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += xf[m, k] * wf[n, k]
                assert abs(y[m, n] - s) <= 1e-12 * max(1.0, abs(s))
        assert np.array_equal(yr, oracle.round_bf16(y))
    x = _bf16_patterns(rng.normal(size=(5, 16)))
    eye = _bf16_patterns(np.eye(16))
    y, yr = oracle.linear_rows(x, eye)
    assert np.array_equal(yr, oracle.decode(x, "bf16"))


def test_silu_closed_forms():
    t = np.linspace(-30, 30, 1201)
    s = oracle.silu(t)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert np.abs(s - oracle.silu(-t) - t).max() < 1e-12
    assert np.abs(s - t * scipy.special.expit(t)).max() < 1e-12


def test_rounded_swiglu():
    # Hand-derived: gate = 1, up = 2 (both exact in bfloat16): silu(1) * 2 =
    # 2 / (1 + e^-1) = 1.46211715726...; the bfloat16 neighbours are
    # 1.4609375 and 1.46875, so the result rounds to 1.4609375.
    x = _bf16_patterns(np.array([[1.0, 0.0]]))
    wg = _bf16_patterns(np.array([[1.0, 0.0]]))
    wu = _bf16_patterns(np.array([[2.0, 5.0]]))
    y, yr, g, u = oracle.swiglu_rows(x, wg, wu)
    assert g[0, 0] == 1.0 and u[0, 0] == 2.0
    assert abs(y[0, 0] - 2.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert yr[0, 0] == 1.4609375
    rng = np.random.default_rng(3)
    x = _bf16_patterns(rng.normal(size=(4, 40)))
    wg = _bf16_patterns(rng.normal(size=(6, 40)) * 0.2)
    wu = _bf16_patterns(rng.normal(size=(6, 40)) * 0.2)
    y, yr, g, u = oracle.swiglu_rows(x, wg, wu)
    assert np.array_equal(g, oracle.linear_rows(x, wg)[1])
    assert np.array_equal(u, oracle.linear_rows(x, wu)[1])
    assert np.array_equal(yr, oracle.round_bf16(g * scipy.special.expit(g) * u))
