"""Pins for the oracle's number formats: OCP e4m3, bf16 rounding, exp/sigmoid/SiLU.

Each primitive is checked against something other than itself: the format's
published named values, torch's own dtype casts, brute-force nearest search,
and fp64 math.
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def ulp_diff(a, b):
    """Distance in fp32 ulps between two finite same-sign floats."""
    return abs(int(f32_bits(a)) - int(f32_bits(b)))


# ---- e4m3 -----------------------------------------------------------------

def test_e4m3_golden_values():
    path = os.path.join(HERE, "golden", "e4m3_ocp_values.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        code, val = line.split()
        v = oracle.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(v)
        else:
            assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val)), code
        n += 1
    assert n >= 10


def test_e4m3_table_matches_torch_cast():
    """Decoding every code agrees with torch.float8_e4m3fn's own decode."""
    table = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    both_nan = np.isnan(table) & np.isnan(ref)
    assert np.array_equal(table[~both_nan], ref[~both_nan])
    assert np.isnan(table).sum() == 2  # 0x7F and 0xFF


def _brute_encode(v, table):
    """Nearest finite e4m3 value by exhaustive search; ties to the even code; sign kept."""
    v = float(np.float32(v))
    a = min(abs(v), 448.0)
    best = None
    for c in range(0x7F):  # non-negative finite codes
        d = abs(float(table[c]) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    c = best[1]
    return c | (0x80 if math.copysign(1.0, v) < 0 else 0)


def _e4m3_midpoints(table):
    pos = np.array([float(table[c]) for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    out = []
    for m in mids:
        f = np.float32(m)
        assert float(f) == m  # e4m3 midpoints are exact in fp32
        out += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    return np.array(out, dtype=np.float32)


def test_e4m3_encode_midpoints_brute_force():
    table = oracle.e4m3_decode_table()
    vals = _e4m3_midpoints(table)
    vals = np.concatenate([vals, -vals, np.array([0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30,
                                                  1e-30, -1e-30], dtype=np.float32)])
    for v in vals:
        assert oracle.e4m3_encode(float(v)) == _brute_encode(v, table), float(v)


def test_e4m3_encode_matches_torch_cast_random():
    """torch's float8_e4m3fn cast rounds to nearest even; inside +-448 it must agree."""
    g = np.random.default_rng(123)
    mags = np.exp(g.uniform(np.log(1e-6), np.log(448.0), 20000)).astype(np.float32)
    vals = (mags * np.where(g.random(20000) < 0.5, -1, 1)).astype(np.float32)
    table = oracle.e4m3_decode_table()
    vals = np.concatenate([vals, _e4m3_midpoints(table)])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    # torch maps values that round to zero to +-0 with the sign kept, as we do
    assert np.array_equal(got, ref)


# ---- bf16 -----------------------------------------------------------------

def test_bf16_rne_matches_torch():
    g = np.random.default_rng(7)
    vals = g.standard_normal(20000).astype(np.float32) * np.float32(100.0)
    # midpoints between adjacent bf16 values and their fp32 neighbours
    base = (g.integers(0x0080, 0x7F00, 3000).astype(np.uint32) << 16)
    mids = (base | 0x8000).view(np.float32)
    vals = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf)), -mids])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_roundtrip_exhaustive():
    """Every finite bf16 pattern survives bf16 -> fp32 -> bf16 unchanged."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    finite = np.isfinite(f)
    back = torch.from_numpy(f[finite]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(back, bits[finite].astype(np.uint16))
    sample = bits[finite][::97]
    for b in sample:
        assert oracle.bf16_rne(float((np.uint32(b) << 16).view(np.float32))) == b


def test_bf16_rne_f64_is_nearest():
    """The fp64 -> bf16 rounding picks the nearest bf16 (ties to even), checked with exact rationals."""
    from fractions import Fraction
    g = np.random.default_rng(11)
    vals = list(g.standard_normal(3000) * 10.0) + [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                                   -(1.0 + 2.0 ** -8), 3.0e-39, 1.0 + 2.0 ** -8 + 2.0 ** -40]
    for d in vals:
        b = oracle.bf16_rne_f64(d)
        v = Fraction(float((np.uint32(b) << 16).view(np.float32)))
        lo = Fraction(float((np.uint32((b - 1) & 0xFFFF) << 16).view(np.float32)))
        hi = Fraction(float((np.uint32((b + 1) & 0xFFFF) << 16).view(np.float32)))
        x = Fraction(d)
        assert abs(v - x) <= abs(lo - x) and abs(v - x) <= abs(hi - x), d
        if abs(v - x) == abs(lo - x) or abs(v - x) == abs(hi - x):
            assert b % 2 == 0, d


# ---- exp / sigmoid / SiLU -----------------------------------------------

def test_exp_ref_accuracy():
    g = np.random.default_rng(5)
    xs = np.concatenate([g.uniform(-80, 80, 20000), g.uniform(-2, 2, 20000),
                         np.array([0.0, 1.0, -1.0, math.log(2), 80.0, -80.0])]).astype(np.float32)
    worst = 0
    for x in xs:
        got = oracle.exp_ref(float(x))
        ref = float(np.float32(math.exp(float(x))))
        worst = max(worst, ulp_diff(got, ref))
    assert worst <= 2, worst


def test_exp_ref_clamps():
    assert oracle.exp_ref(1000.0) == oracle.exp_ref(80.0)
    assert oracle.exp_ref(-1000.0) == oracle.exp_ref(-80.0)
    assert oracle.exp_ref(0.0) == 1.0


def test_sigmoid_accuracy_and_symmetry():
    g = np.random.default_rng(6)
    worst = 0
    for x in g.uniform(-20, 20, 20000).astype(np.float32):
        got = oracle.sigmoid(float(x))
        ref = float(np.float32(1.0 / (1.0 + math.exp(-float(x)))))
        worst = max(worst, ulp_diff(got, ref))
    assert worst <= 3, worst
    assert oracle.sigmoid(0.0) == 0.5


def test_silu_mul_bf16_close_to_exact():
    """h = bf16(SiLU(g) * u) is the correctly rounded value or one bf16 step from it."""
    g = np.random.default_rng(8)
    gs = g.standard_normal(20000).astype(np.float32) * np.float32(2.0)
    us = g.standard_normal(20000).astype(np.float32) * np.float32(2.0)
    exact = 0
    for a, b in zip(gs, us):
        h = oracle.silu_mul_bf16(float(a), float(b))
        ref = float(a) / (1.0 + math.exp(-float(a))) * float(b)
        rb = oracle.bf16_rne_f64(ref)
        assert abs(int(h) - int(rb)) <= 1 or (ref == 0.0), (a, b)
        exact += int(h) == int(rb)
    assert exact >= 0.99 * len(gs)


def test_math_vec_is_the_scalar_definitions():
    """The array form used for dense device comparisons evaluates exactly the
    pinned scalar exp_ref and sigmoid, and SiLU as x / (1 + exp_ref(-x))."""
    g = np.random.default_rng(3)
    x = np.concatenate([np.linspace(-90, 90, 2001), g.uniform(-88, 88, 2000),
                        [0.0, -0.0, 1e-30, -1e-30]]).astype(np.float32)
    e, sg, sl = oracle.math_vec(x)
    for v, a, b, c in zip(x, e, sg, sl):
        assert np.float32(oracle.exp_ref(float(v))) == a
        assert np.float32(oracle.sigmoid(float(v))) == b
        d = np.float32(1.0) + np.float32(oracle.exp_ref(float(-v)))
        assert np.float32(v) / d == c or (np.isnan(c) and np.isnan(np.float32(v) / d))
