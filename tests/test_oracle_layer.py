"""Pins for the oracle's quantisation, grouped GEMM, activation, combine and whole layer.

- dynamic scales: bitwise amax/448, round trip within half an e4m3 step,
  codes equal to torch's own float8 cast;
- grouped GEMM: an exact-arithmetic case that must be bit exact (and whose
  mutation, scale_a indexed by expert, must fail), and agreement with an fp64
  numpy matmul of the dequantised operands;
- combine: nearest bf16 of the fp64 weighted sum;
- layer: the dense per-token loop equals the permuted path bit for bit; the
  tiny layer is within the FP8 quantisation budget of an unquantised fp64
  layer; zero-token experts are never read; the routed scaling factor scales
  the output once.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

E4M3_TABLE = None


def table():
    global E4M3_TABLE
    if E4M3_TABLE is None:
        E4M3_TABLE = oracle.e4m3_decode_table().astype(np.float64)
    return E4M3_TABLE


def bf(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def e4m3_half_step(q):
    """Half the gap between |q| and the next e4m3 magnitude (q already decoded)."""
    a = np.abs(q)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


# ---- dynamic activation quantisation ----------------------------------------

@pytest.mark.parametrize("mode", [W.ACT_PER_TOKEN, W.ACT_PER_GROUP, W.ACT_PER_TENSOR])
def test_pre_reorder_quant_scales_and_roundtrip(mode):
    g = np.random.default_rng(20 + mode)
    T, H, K = 40, 320, 3
    x = g.standard_normal((T, H)).astype(np.float32)
    x *= (2.0 ** (np.arange(T) % 7 - 3)).astype(np.float32)[:, None]   # very different rows
    x[5] = 0.0                                                         # all-zero token
    xb = W.to_bf16_bits(x)
    ids = np.stack([g.permutation(8)[:K] for _ in range(T)]).astype(np.int32)
    m_cap = T * K
    s2d, d2s, seg = oracle.permute(ids, 0, 8, m_cap)
    a_q, a_s = oracle.pre_reorder_quant(xb, s2d, K, mode, m_cap)
    xf = bf(xb)
    G = -(-H // 128)
    dec = table()[a_q]
    for r in range(m_cap):
        t = d2s[r] // K
        row = xf[t]
        if mode == W.ACT_PER_TENSOR:
            amaxes = [np.float32(np.abs(xf).max())] * G
            scales = [a_s[0]] * G
        elif mode == W.ACT_PER_TOKEN:
            amaxes = [np.float32(np.abs(row).max())] * G
            scales = [a_s[r]] * G
        else:
            amaxes = [np.float32(np.abs(row[q * 128:(q + 1) * 128]).max()) for q in range(G)]
            scales = list(a_s[r * G:(r + 1) * G])
        for q in range(G):
            am = max(amaxes[q], np.float32(1e-10))
            assert np.float32(scales[q]) == np.float32(am) / np.float32(448.0)
            sl = slice(q * 128, (q + 1) * 128)
            err = np.abs(dec[r, sl] * float(scales[q]) - row[sl])
            bound = (e4m3_half_step(row[sl] / float(scales[q])) * float(scales[q])) * (1 + 1e-6) + 1e-30
            assert np.all(err <= bound), (r, q)
            inv = np.float32(448.0) / np.float32(am)
            ref = W.to_e4m3_codes((row[sl].astype(np.float32) * inv).astype(np.float32))
            assert np.array_equal(a_q[r, sl], ref)
    assert np.all(a_q[s2d[5 * K:6 * K]] == 0)


# ---- grouped GEMM: exact-arithmetic case ------------------------------------

def _exact_gemm_case(act_quant, w_quant, seed=0, counts=(37, 0, 90, 21), N=256, K=256, extra=11):
    g = np.random.default_rng(30 + seed)
    counts = np.asarray(counts)
    E_l = len(counts)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m_cap = int(seg[-1]) + extra
    codes = np.array([0x38, 0xB8, 0x00], dtype=np.uint8)      # +1, -1, 0
    a_q = codes[g.integers(0, 3, (m_cap, K))]
    b_q = codes[g.integers(0, 3, (E_l, N, K))]
    KB, NB = K // 128, N // 128
    r = np.arange(m_cap)
    if act_quant == W.ACT_PER_TENSOR:
        sa = np.array([0.25], np.float32)
        sa_full = np.full((m_cap, K), 0.25)
    elif act_quant == W.ACT_PER_TOKEN:
        sa = (2.0 ** (r % 7 - 3)).astype(np.float32)
        sa_full = np.repeat(sa[:, None].astype(np.float64), K, axis=1)
    else:
        sa = (2.0 ** ((r[:, None] + np.arange(KB)[None, :]) % 5 - 2)).astype(np.float32)
        sa_full = np.repeat(sa.astype(np.float64), 128, axis=1)
        sa = sa.reshape(-1)
    if w_quant == W.W_PER_EXPERT:
        sb = (2.0 ** (np.arange(E_l) % 3 - 1)).astype(np.float32)
        sb_full = np.broadcast_to(sb.astype(np.float64)[:, None, None], (E_l, N, K))
    elif w_quant == W.W_PER_CHANNEL:
        sb = (2.0 ** ((np.arange(E_l)[:, None] + np.arange(N)[None, :]) % 5 - 2)).astype(np.float32)
        sb_full = np.repeat(sb.astype(np.float64)[:, :, None], K, axis=2)
        sb = sb.reshape(-1)
    else:
        idx = np.arange(E_l)[:, None, None] + np.arange(NB)[None, :, None] + np.arange(KB)[None, None, :]
        sb = (2.0 ** (idx % 3 - 1)).astype(np.float32)
        sb_full = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=1), 128, axis=2)
        sb = sb.reshape(-1)
    A = table()[a_q] * sa_full
    expect = np.zeros((m_cap, N), dtype=np.uint16)
    for e in range(E_l):
        rows = slice(seg[e], seg[e + 1])
        B = table()[b_q[e]] * sb_full[e]
        exact = A[rows] @ B.T                      # every partial sum is exact in fp32
        expect[rows] = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16) \
            .view(torch.int16).numpy().view(np.uint16)
    return a_q, sa, b_q, sb, seg, expect, m_cap


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL),
                                               (W.ACT_PER_GROUP, W.W_BLOCK),
                                               (W.ACT_PER_GROUP, W.W_PER_CHANNEL),
                                               (W.ACT_PER_TOKEN, W.W_BLOCK)])
def test_grouped_gemm_exact_case(act_quant, w_quant):
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant)
    c = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    assert np.array_equal(c[:M], expect[:M])


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TOKEN, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL),
                                               (W.ACT_PER_GROUP, W.W_BLOCK)])
def test_grouped_gemm_mutation_scale_a_by_expert_is_caught(act_quant, w_quant):
    """The defect the row indexing fixes (scale_a read at the expert id) must fail the pin."""
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant)
    c = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg,
                            flags=oracle.FLAG_SCALE_A_BY_EXPERT)
    M = seg[-1]
    assert not np.array_equal(c[:M], expect[:M])


def test_grouped_gemm_matches_fp64_matmul():
    g = np.random.default_rng(40)
    M, N, K = 70, 96, 384
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (M, K))]
    b_q = finite[g.integers(0, len(finite), (1, N, K))]
    sa = g.uniform(0.001, 0.01, M).astype(np.float32)
    sb = g.uniform(0.0005, 0.002, N).astype(np.float32)
    seg = np.array([0, M], np.int32)
    c = oracle.grouped_gemm(a_q, sa, W.ACT_PER_TOKEN, b_q, sb, W.W_PER_CHANNEL, seg)
    A = table()[a_q] * sa.astype(np.float64)[:, None]
    B = table()[b_q[0]] * sb.astype(np.float64)[:, None]
    ref = A @ B.T
    bound = np.abs(A) @ np.abs(B).T * (K * 2.0 ** -23) + np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(bf(c) - ref) <= bound)


def test_grouped_gemm_k_tail_and_empty_experts():
    """K not a multiple of 128 and experts with zero rows."""
    g = np.random.default_rng(41)
    E_l, N, K = 3, 40, 80
    seg = np.array([0, 0, 13, 13], np.int32)
    a_q = g.integers(0, 0x7E, (16, K)).astype(np.uint8)
    b_q = g.integers(0, 0x7E, (E_l, N, K)).astype(np.uint8)
    sa = np.full(16, 0.01, np.float32)
    sb = np.full(E_l, 0.01, np.float32)
    c = oracle.grouped_gemm(a_q, sa, W.ACT_PER_TOKEN, b_q, sb, W.W_PER_EXPERT, seg)
    A = table()[a_q[:13]] * 0.01
    ref = A @ (table()[b_q[1]] * 0.01).T
    assert np.all(np.abs(bf(c[:13]) - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-9)
    assert np.all(c[13:] == 0)



_MODE_PAIRS = [(W.ACT_PER_TENSOR, W.W_PER_EXPERT), (W.ACT_PER_TOKEN, W.W_PER_EXPERT),
               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL), (W.ACT_PER_GROUP, W.W_BLOCK),
               (W.ACT_PER_GROUP, W.W_PER_CHANNEL), (W.ACT_PER_TOKEN, W.W_BLOCK)]


@pytest.mark.parametrize("act_quant,w_quant", _MODE_PAIRS)
def test_grouped_gemm_rows_reproduces_exact_case(act_quant, w_quant):
    """The sampled-row GEMM reproduces the exact-arithmetic case row by row (every
    row of every segment, the padding rows past M as zeros)."""
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant)
    rows = np.arange(m_cap)
    c = oracle.grouped_gemm_rows(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows)
    M = int(seg[-1])
    assert np.array_equal(c[:M], expect[:M])
    assert np.all(c[M:] == 0)


@pytest.mark.parametrize("act_quant,w_quant", _MODE_PAIRS)
def test_grouped_gemm_rows_equals_full_gemm_at_boundaries(act_quant, w_quant):
    """Random finite codes and scales on ragged segments with empty experts: the
    rows on both sides of every segment boundary, random interior rows and rows
    at or past M equal the whole-matrix oracle's rows bit for bit (rows outside
    every segment are zeros there too). A wrong row-to-expert lookup at a
    boundary or a scale read at the wrong row breaks the equality."""
    g = np.random.default_rng(60 + 7 * act_quant + w_quant)
    N, K = 160, 384
    counts = np.array([0, 5, 1, 0, 17, 2, 0, 9])
    E_l = len(counts)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(seg[-1])
    m_cap = M + 6
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (m_cap, K))]
    b_q = finite[g.integers(0, len(finite), (E_l, N, K))]
    sa = g.uniform(0.5, 2.0, W.a_scale_numel(act_quant, m_cap, K)).astype(np.float32)
    sb = g.uniform(0.5, 2.0, W.b_scale_numel(w_quant, E_l, N, K)).astype(np.float32)
    full = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    edges = [r for e in range(E_l) if counts[e] > 0 for r in (seg[e], seg[e + 1] - 1)]
    rows = np.array(sorted(set(edges)) + list(g.integers(0, M, 6)) + [M, M + 1, m_cap - 1],
                    dtype=np.int64)
    c = oracle.grouped_gemm_rows(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows)
    assert np.array_equal(c, full[rows])
    assert np.all(c[-3:] == 0)
    # the rows really are distinct data (a lookup that returned the wrong expert
    # or scale row would not go unnoticed)
    assert len({bytes(r) for r in c[:len(edges)]}) == len(edges)

# ---- activation + requant -----------------------------------------------------

@pytest.mark.parametrize("mode", [W.ACT_PER_TOKEN, W.ACT_PER_GROUP, W.ACT_PER_TENSOR])
def test_act_requant_properties(mode):
    g = np.random.default_rng(50 + mode)
    m_cap, I = 60, 192
    seg = np.array([0, 20, 20, 51], np.int32)
    gu = W.to_bf16_bits(g.standard_normal((m_cap, 2 * I)).astype(np.float32) * np.float32(2.0))
    a_q, a_s = oracle.act_requant(gu, seg, mode)
    M = seg[-1]
    f = bf(gu)
    h = np.array([[oracle.silu_mul_bf16(f[r, i], f[r, I + i]) for i in range(I)] for r in range(M)],
                 dtype=np.uint16)
    hf = bf(h)
    exact = f[:M, :I] / (1.0 + np.exp(-f[:M, :I])) * f[:M, I:]
    assert np.all(np.abs(hf - exact) <= np.abs(exact) * 2.0 ** -7 + 1e-30)
    G = -(-I // 128)
    dec = table()[a_q]
    for r in range(M):
        for q in range(G):
            sl = slice(q * 128, min((q + 1) * 128, I))
            if mode == W.ACT_PER_TENSOR:
                am, s = np.float32(np.abs(hf).max()), a_s[0]
            elif mode == W.ACT_PER_TOKEN:
                am, s = np.float32(np.abs(hf[r]).max()), a_s[r]
            else:
                am, s = np.float32(np.abs(hf[r, sl]).max()), a_s[r * G + q]
            assert np.float32(s) == max(am, np.float32(1e-10)) / np.float32(448.0)
            err = np.abs(dec[r, sl] * float(s) - hf[r, sl])
            assert np.all(err <= e4m3_half_step(hf[r, sl] / float(s)) * float(s) * (1 + 1e-6) + 1e-30)


# ---- combine -----------------------------------------------------------------

def test_post_reorder_nearest_bf16_of_fp64_sum():
    g = np.random.default_rng(60)
    T, H, K = 33, 64, 4
    ids = np.stack([g.permutation(10)[:K] for _ in range(T)]).astype(np.int32)
    s2d, d2s, seg = oracle.permute(ids, 2, 5, T * K)
    M = seg[-1]
    down = W.to_bf16_bits(g.standard_normal((T * K, H)).astype(np.float32))
    w = g.uniform(0, 1, (T, K)).astype(np.float32)
    out = oracle.post_reorder(down, s2d, w, T, K)
    d = bf(down)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(K):
            r = s2d[t * K + j]
            if r >= 0:
                acc += float(w[t, j]) * d[r]
        o = bf(out[t])
        assert np.all(np.abs(o - acc) <= np.abs(acc) * 2.0 ** -8 * (1 + 1e-9) + 1e-38)
        if np.all(s2d[t * K:(t + 1) * K] < 0):
            assert np.all(out[t] == 0)
    assert M < T * K


# ---- whole layer ----------------------------------------------------------------

def small_cfg(mode_name):
    base = dict(T=50, H=256, I=192, E=16, topk=4)
    if mode_name == "ep_sigmoid_token_channel":
        return W.MoEConfig(name=mode_name, num_local=6, expert_start=5, score_fn=W.SCORE_SIGMOID,
                           n_group=4, topk_group=2, rsf=2.5, use_bias=True,
                           act_quant=W.ACT_PER_TOKEN, w_quant=W.W_PER_CHANNEL, **base)
    if mode_name == "softmax_tensor_expert":
        return W.MoEConfig(name=mode_name, num_local=16, score_fn=W.SCORE_SOFTMAX,
                           act_quant=W.ACT_PER_TENSOR, w_quant=W.W_PER_EXPERT, **base)
    if mode_name == "skew_group_block":
        return W.MoEConfig(name=mode_name, num_local=16, score_fn=W.SCORE_SOFTMAX,
                           act_quant=W.ACT_PER_GROUP, w_quant=W.W_BLOCK, zipf_skew=1.2,
                           cold_experts=3, **base)
    raise KeyError(mode_name)


LAYER_CASES = ["ep_sigmoid_token_channel", "softmax_tensor_expert", "skew_group_block"]


@pytest.mark.parametrize("name", LAYER_CASES)
def test_dense_equals_permuted_bitwise(name):
    cfg = small_cfg(name)
    inp = W.gen_layer_inputs(cfg, seed=3)
    res = oracle.layer(inp)
    dense = oracle.dense_layer(inp.x, res["ids"], res["weights"], cfg.I, cfg.expert_start,
                               cfg.num_local, cfg.act_quant, inp.w13, inp.w13_scale, inp.w2,
                               inp.w2_scale, cfg.w_quant)
    assert np.array_equal(dense, res["out"])


def test_dense_equals_permuted_tiny():
    cfg = W.CONFIGS["tiny"]
    inp = W.gen_layer_inputs(cfg)
    res = oracle.layer(inp)
    dense = oracle.dense_layer(inp.x, res["ids"], res["weights"], cfg.I, cfg.expert_start,
                               cfg.num_local, cfg.act_quant, inp.w13, inp.w13_scale, inp.w2,
                               inp.w2_scale, cfg.w_quant)
    assert np.array_equal(dense, res["out"])


def _fp64_layer(inp, ids, weights):
    """Unquantised activations, dequantised weights, fp64 everywhere."""
    cfg = inp.cfg
    x = bf(inp.x)
    out = np.zeros((cfg.T, cfg.H))
    t13 = table()[inp.w13]
    t2 = table()[inp.w2]
    for e in range(cfg.num_local):
        s13 = W._expand_scales(inp.w13_scale[e].reshape(-1 if cfg.w_quant != W.W_BLOCK else
                                                          (-(-2 * cfg.I // 128), -(-cfg.H // 128))),
                               cfg.w_quant, 2 * cfg.I, cfg.H)
        s2 = W._expand_scales(inp.w2_scale[e].reshape(-1 if cfg.w_quant != W.W_BLOCK else
                                                        (-(-cfg.H // 128), -(-cfg.I // 128))),
                              cfg.w_quant, cfg.H, cfg.I)
        w13 = t13[e] * s13
        w2 = t2[e] * s2
        for t in range(cfg.T):
            for j in range(cfg.topk):
                if ids[t, j] - cfg.expert_start != e:
                    continue
                gu = w13 @ x[t]
                gg, uu = gu[:cfg.I], gu[cfg.I:]
                h = gg / (1.0 + np.exp(-gg)) * uu
                out[t] += float(weights[t, j]) * (w2 @ h)
    return out


def test_tiny_layer_within_fp8_budget_of_fp64():
    cfg = W.CONFIGS["tiny"]
    inp = W.gen_layer_inputs(cfg)
    res = oracle.layer(inp)
    ref = _fp64_layer(inp, res["ids"], res["weights"])
    got = bf(res["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 0.06, rel


def test_layer_mutation_scale_a_by_expert_is_caught():
    """With strongly different token magnitudes, reading scale_a at the expert id breaks the layer."""
    cfg = W.CONFIGS["tiny"]
    inp = W.gen_layer_inputs(cfg)
    x = bf(inp.x) * (2.0 ** (np.arange(cfg.T) % 5 - 2))[:, None]
    inp = dataclasses.replace(inp, x=W.to_bf16_bits(x.astype(np.float32)))
    good = oracle.layer(inp)
    bad = oracle.layer(inp, flags=oracle.FLAG_SCALE_A_BY_EXPERT)
    ref = _fp64_layer(inp, good["ids"], good["weights"])
    rel_good = np.linalg.norm(bf(good["out"]) - ref) / np.linalg.norm(ref)
    rel_bad = np.linalg.norm(bf(bad["out"]) - ref) / np.linalg.norm(ref)
    assert rel_good < 0.06 and rel_bad > 0.3, (rel_good, rel_bad)


def test_zero_token_experts_never_read():
    cfg = small_cfg("skew_group_block")
    inp = W.gen_layer_inputs(cfg, seed=5)
    res = oracle.layer(inp)
    seg = res["seg_indptr"]
    empty = [e for e in range(cfg.num_local) if seg[e] == seg[e + 1]]
    assert len(empty) >= 1
    w13, w2 = inp.w13.copy(), inp.w2.copy()
    w13[empty] = 0x7F
    w2[empty] = 0x7F
    s13, s2 = inp.w13_scale.copy(), inp.w2_scale.copy()
    s13[empty] = np.nan
    s2[empty] = np.nan
    res2 = oracle.layer(dataclasses.replace(inp, w13=w13, w2=w2, w13_scale=s13, w2_scale=s2))
    assert np.array_equal(res2["out"], res["out"])


def test_routed_scaling_factor_scales_output_once():
    cfg = small_cfg("ep_sigmoid_token_channel")
    inp = W.gen_layer_inputs(cfg, seed=7)
    o25 = bf(oracle.layer(inp)["out"])
    o1 = bf(oracle.layer(dataclasses.replace(inp, cfg=dataclasses.replace(cfg, rsf=1.0)))["out"])
    assert np.all(np.abs(o25 - 2.5 * o1) <= np.abs(o25) * 2.0 ** -7 + 1e-30)
    assert np.abs(o25).max() > 0
