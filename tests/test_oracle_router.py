"""Pins of the oracle's router projection (logits the gate scores), against
things other than itself: numpy's fp64 matrix product of the same bf16 values,
exact rational arithmetic on a tiny case, unit-vector rows that pick columns of
x, and exact scaling by a power of two."""
from fractions import Fraction

import numpy as np

import oracle
import workloads as W


def _bits(a):
    return W.to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_router_matches_numpy_fp64_product():
    g = np.random.default_rng(0)
    x = _bits(g.standard_normal((37, 200)))
    wg = _bits(g.standard_normal((12, 200)) * 0.02)
    got = oracle.router_logits(x, wg)
    ref = W.bf16_bits_to_f32(x).astype(np.float64) @ W.bf16_bits_to_f32(wg).astype(np.float64).T
    ref32 = ref.astype(np.float32)
    # both are fp64 sums of exact products rounded once to fp32; summation order
    # differs, so allow one fp32 step where the fp64 sums straddle a boundary
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
    assert np.mean(got == ref32) > 0.999


def test_router_exact_rational_tiny():
    g = np.random.default_rng(1)
    x = _bits(g.standard_normal((3, 16)))
    wg = _bits(g.standard_normal((4, 16)))
    got = oracle.router_logits(x, wg)
    xf, wf = W.bf16_bits_to_f32(x), W.bf16_bits_to_f32(wg)
    for t in range(3):
        for e in range(4):
            exact = sum(Fraction(float(xf[t, h])) * Fraction(float(wf[e, h])) for h in range(16))
            r = np.float32(float(exact))
            assert abs(Fraction(float(got[t, e])) - exact) <= Fraction(float(np.spacing(np.abs(r)))) / 2 * 1.000001


def test_router_unit_rows_pick_columns():
    g = np.random.default_rng(2)
    H, E = 64, 8
    x = _bits(g.standard_normal((5, H)))
    cols = g.choice(H, E, replace=False)
    wg = np.zeros((E, H), np.float32)
    wg[np.arange(E), cols] = 1.0
    got = oracle.router_logits(x, _bits(wg))
    assert np.array_equal(got, W.bf16_bits_to_f32(x)[:, cols])


def test_router_power_of_two_scaling():
    g = np.random.default_rng(3)
    x = _bits(g.standard_normal((9, 96)))
    wg = g.standard_normal((8, 96)).astype(np.float32) * 0.02
    a = oracle.router_logits(x, _bits(wg))
    b = oracle.router_logits(x, _bits(wg * 4))
    assert np.array_equal(b, a * 4)
