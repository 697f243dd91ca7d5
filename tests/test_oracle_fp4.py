"""Pins of the MXFP4-weight grouped GEMM in the oracle.

- the E2M1 decode against the OCP MX element table (tests/golden);
- E8M0 scale special points;
- a hand-worked two-block case (tests/golden/mxfp4_gemm_hand.txt) that fixes
  the nibble order and the 32-element block index;
- an exact reduction to the FP8 grouped GEMM oracle (pinned on its own): when
  every weight row has one block scale, MXFP4 values are e4m3 values and the
  block scale becomes a per-channel factor, so both must give the same bits;
- the same reduction for the whole layer.
"""
import dataclasses
import os

import numpy as np
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_decode_matches_ocp_table():
    rows = _fixture("e2m1_ocp_values.txt")
    assert len(rows) == 16
    for code, value in rows:
        v = oracle.e2m1_value(int(code, 2))
        assert v == float(value) and np.signbit(v) == value.startswith("-"), code


def test_e8m0_points():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def _pack(nib):
    """[.., K] nibbles -> [.., K/2] bytes, element k in byte k/2, low nibble for even k."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def test_hand_worked_two_blocks():
    K, N = 64, 2
    a = np.zeros((1, K), dtype=np.float32)
    a[0, 3], a[0, 40] = 1.0, 2.0
    a_q = W.to_e4m3_codes(a)
    nib = np.zeros((1, N, K), dtype=np.uint8)
    nib[0, 0, 3], nib[0, 0, 40] = 0b0011, 0b0110
    nib[0, 1, 3], nib[0, 1, 40] = 0b1001, 0b0111
    e8m0 = np.array([[[127, 129], [126, 127]]], dtype=np.uint8)
    c = oracle.grouped_gemm_mxfp4(a_q, np.ones(1, np.float32), W.ACT_PER_TOKEN, _pack(nib), e8m0,
                                  np.ones(1, np.float32), W.W_PER_EXPERT, np.array([0, 1], np.int32))
    want = {int(n): float(v) for n, v in _fixture("mxfp4_gemm_hand.txt")}
    got = W.bf16_bits_to_f32(c[0])
    for n in range(N):
        assert got[n] == want[n], (n, got[n], want[n])


def _e2m1_literal():
    """Value of each nibble from the OCP table fixture (not from the oracle)."""
    return np.array([float(v) for _, v in sorted(_fixture("e2m1_ocp_values.txt"),
                                                   key=lambda r: int(r[0], 2))], dtype=np.float32)


def _fp4_to_fp8(nib, e8m0_row, factor, w_quant):
    """MXFP4 weights with one block scale per row -> e4m3 codes and per-channel
    scales of the same values (E2M1 values are exact in e4m3)."""
    vals = _e2m1_literal()[nib]
    codes = W.to_e4m3_codes(vals)
    assert np.array_equal(torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy(), vals)
    E, N, _ = nib.shape
    f = np.broadcast_to(factor.reshape(E, -1), (E, N)) if w_quant == W.W_PER_EXPERT else factor.reshape(E, N)
    scale = (np.ldexp(np.float32(1.0), e8m0_row.astype(np.int32) - 127).astype(np.float32) * f).astype(np.float32)
    return codes, scale.reshape(E, N)


def test_reduces_to_fp8_gemm_with_one_block_scale_per_row():
    g = np.random.default_rng(7)
    E, N, K, M = 3, 48, 96, 37
    for w_quant in (W.W_PER_EXPERT, W.W_PER_CHANNEL):
        for act_quant in (W.ACT_PER_TENSOR, W.ACT_PER_TOKEN):
            nib = g.integers(0, 16, size=(E, N, K), dtype=np.uint8)
            e8m0_row = g.integers(120, 131, size=(E, N)).astype(np.uint8)
            e8m0 = np.repeat(e8m0_row[:, :, None], K // 32, axis=2)
            factor = g.uniform(0.5, 2.0, size=(E, 1 if w_quant == W.W_PER_EXPERT else N)).astype(np.float32)
            a_q = W.to_e4m3_codes(g.standard_normal((M, K)).astype(np.float32) * 40)
            sa = (g.uniform(0.01, 0.1, size=1 if act_quant == W.ACT_PER_TENSOR else M)).astype(np.float32)
            seg = np.array([0, 10, 10, M], dtype=np.int32)  # expert 1 empty
            c4 = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, _pack(nib), e8m0, factor, w_quant, seg)
            codes, scale = _fp4_to_fp8(nib, e8m0_row, factor, w_quant)
            c8 = oracle.grouped_gemm(a_q, sa, act_quant, codes, scale, W.W_PER_CHANNEL, seg)
            assert np.array_equal(c4, c8), (w_quant, act_quant)
            rows = np.array([0, 9, 10, 36, 5], dtype=np.int64)
            assert np.array_equal(
                oracle.grouped_gemm_mxfp4_rows(a_q, sa, act_quant, _pack(nib), e8m0, factor, w_quant, seg, rows),
                c4[rows])


def test_block_scales_differ_from_row_scale():
    """With per-block scales that differ, the result is not the one-scale result
    (guards against a block index that always reads block 0)."""
    g = np.random.default_rng(8)
    E, N, K, M = 1, 16, 128, 8
    nib = g.integers(1, 8, size=(E, N, K), dtype=np.uint8)
    e8m0 = np.full((E, N, K // 32), 127, dtype=np.uint8)
    a_q = W.to_e4m3_codes(np.abs(g.standard_normal((M, K))).astype(np.float32) + 0.5)
    sa = np.ones(M, np.float32)
    seg = np.array([0, M], np.int32)
    base = W.bf16_bits_to_f32(oracle.grouped_gemm_mxfp4(a_q, sa, 1, _pack(nib), e8m0, np.ones((1, 1), np.float32), 0, seg))
    e8m0[:, :, 3] = 128
    up = W.bf16_bits_to_f32(oracle.grouped_gemm_mxfp4(a_q, sa, 1, _pack(nib), e8m0, np.ones((1, 1), np.float32), 0, seg))
    assert np.all(up > base)  # positive products in the last block doubled


def test_layer_reduces_to_fp8_layer():
    cfg4 = W.MoEConfig(name="small_fp4", T=24, H=128, I=64, E=8, topk=2, num_local=5, expert_start=2,
                       score_fn=W.SCORE_SOFTMAX, act_quant=W.ACT_PER_TOKEN, w_quant=W.W_PER_EXPERT,
                       w_fp4=True)
    inp4 = W.gen_layer_inputs(cfg4, seed=3)
    # one block scale per weight row
    e13 = np.repeat(inp4.w13_e8m0[:, :, :1], inp4.w13_e8m0.shape[2], axis=2)
    e2 = np.repeat(inp4.w2_e8m0[:, :, :1], inp4.w2_e8m0.shape[2], axis=2)
    inp4 = dataclasses.replace(inp4, w13_e8m0=e13, w2_e8m0=e2)

    def unpack(p):
        out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
        out[..., 0::2], out[..., 1::2] = p & 15, p >> 4
        return out

    c13, s13 = _fp4_to_fp8(unpack(inp4.w13), e13[:, :, 0], inp4.w13_scale, W.W_PER_EXPERT)
    c2, s2 = _fp4_to_fp8(unpack(inp4.w2), e2[:, :, 0], inp4.w2_scale, W.W_PER_EXPERT)
    cfg8 = dataclasses.replace(cfg4, w_fp4=False, w_quant=W.W_PER_CHANNEL)
    inp8 = dataclasses.replace(inp4, cfg=cfg8, w13=c13, w13_scale=s13, w2=c2, w2_scale=s2,
                               w13_e8m0=None, w2_e8m0=None)
    r4, r8 = oracle.layer(inp4), oracle.layer(inp8)
    for key in ("c13", "a2", "a2_scale", "c2", "out"):
        assert np.array_equal(r4[key], r8[key]), key
