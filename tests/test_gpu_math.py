"""The library's fixed-sequence device math (exp_fixed, sigmoid_fixed,
silu_fixed) against the CPU oracle's exp_ref, sigmoid and SiLU, bit for bit on
a dense sample: expert ids (through sigmoid scoring) and FP8 codes (through
SiLU) are compared bit for bit only because both sides evaluate the same fp32
operation sequence, and one ulp of drift would flip near-tied selections."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_grouped_gemm_select_amd import _build
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def device_math(x):
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.moe_probe_math.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    xd = G.up(np.ascontiguousarray(x, np.float32))
    outs = [torch.empty_like(xd) for _ in range(3)]
    rc = lib.moe_probe_math(xd.data_ptr(), xd.numel(), *[o.data_ptr() for o in outs],
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def test_exp_sigmoid_silu_bitwise_on_a_dense_sample():
    """4M evenly spaced values over [-80, 80] (steps of about 4e-5), 1M random
    fp32 bit patterns in [-88, 88], every fp32 in [1, 1 + 2^-10) and around the
    clamp points: exp and sigmoid bit-exact everywhere; SiLU bit-exact except
    below |x| = 2^-102, where the device division may differ in the last place
    of a value under 2^-102 and keeps the sign."""
    g = np.random.default_rng(17)
    dense = np.linspace(-80.0, 80.0, 1 << 22, dtype=np.float32)
    rnd = g.uniform(-88.0, 88.0, 1 << 20).astype(np.float32)
    ones = (np.arange(1 << 13, dtype=np.uint32) + np.float32(1.0).view(np.uint32)).view(np.float32)
    edges = np.array([0.0, -0.0, 80.0, -80.0, np.nextafter(np.float32(80), np.float32(0)),
                      np.nextafter(np.float32(-80), np.float32(0)), 80.001, -80.001, 88.7, -87.3,
                      1e-30, -1e-30, 2.0 ** -126, -(2.0 ** -126), 2.0 ** -102, -(2.0 ** -102)],
                     dtype=np.float32)
    x = np.concatenate([dense, rnd, ones, -ones, edges])
    print(f"device math on {len(x)} values", flush=True)
    e_g, s_g, l_g = device_math(x)
    e_r, s_r, l_r = oracle.math_vec(x)
    for name, a, b in (("exp", e_g, e_r), ("sigmoid", s_g, s_r)):
        bad = a.view(np.uint32) != b.view(np.uint32)
        assert not bad.any(), f"{name}: {int(bad.sum())} values differ, first at x={x[bad][:4]}"
    tiny = np.abs(x) < 2.0 ** -102
    bad = (l_g.view(np.uint32) != l_r.view(np.uint32)) & ~tiny
    assert not bad.any(), f"silu: {int(bad.sum())} values differ, first at x={x[bad][:4]}"
    assert np.all(np.signbit(l_g[tiny]) == np.signbit(l_r[tiny]))
    assert np.all(np.abs(l_g[tiny].astype(np.float64) - l_r[tiny]) <= np.spacing(np.abs(l_r[tiny])))
