"""GPU parity of the grouped GEMM with MXFP4 expert weights (moe_grouped_gemm_mxfp4)
against the oracle: an exact case (every product and partial sum exact, so the
bits must agree), ragged random cases with empty experts and partial tiles in
both directions, and the full DeepSeek-V3 shares on sampled rows in the
benchmark's launch configuration. The whole layer with FP4 weights is covered in
test_gpu_layer.py."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _seg(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _fp4_weights(g, E, N, K, e8m0_lo=120, e8m0_hi=131):
    nib = g.integers(0, 16, size=(E, N, K), dtype=np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    e8m0 = g.integers(e8m0_lo, e8m0_hi, size=(E, N, K // 32)).astype(np.uint8)
    return packed, e8m0


def abs_products_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg, rows):
    """sum_k |a_hat[r,k] * b_hat[e,n,k]| (fp64) for the given rows."""
    table = np.abs(oracle.e4m3_decode_table().astype(np.float64))
    sa = np.asarray(sa, np.float64).reshape(-1)
    sb = np.asarray(sb, np.float64).reshape(-1)
    N = b_fp4.shape[1]
    out = np.zeros((len(rows), N))
    cache = {}
    for i, r in enumerate(rows):
        e = int(np.searchsorted(seg, r, side="right") - 1)
        if e not in cache:
            f = abs(sb[e]) if w_quant == W.W_PER_EXPERT else np.abs(sb[e * N:(e + 1) * N])[:, None]
            cache[e] = G.fp4_abs_values(b_fp4[e], b_e8m0[e]) * f
        a = table[a_q[r]] * abs(sa[0] if act_quant == W.ACT_PER_TENSOR else sa[r])
        out[i] = cache[e] @ a
    return out


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL)])
@pytest.mark.parametrize("K", [384, 768])  # 128-deep and 256-deep K steps
def test_mxfp4_gemm_exact_case(act_quant, w_quant, K):
    """Activations in {-1, 0, 1}, weights in {0, +-0.5, +-1, +-2} times block
    scales 2^-1 or 2^0, and power-of-two factors: every product and partial sum
    is a multiple of 2^-2 below 2^10, exact in fp32 and inside the MFMA's
    internal precision, so the bf16 results must be bit-identical."""
    g = np.random.default_rng(11)
    counts = [70, 0, 129, 3]
    seg = _seg(counts)
    m_cap, N = int(seg[-1]) + 5, 272
    E = len(counts)
    a_q = W.to_e4m3_codes(g.integers(-1, 2, size=(m_cap, K)).astype(np.float32))
    nib = np.array([0, 1, 2, 4, 9, 10, 12], np.uint8)[g.integers(0, 7, size=(E, N, K))]
    b_fp4 = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    b_e8m0 = g.integers(126, 128, size=(E, N, K // 32)).astype(np.uint8)
    sa = np.ldexp(1.0, g.integers(-2, 3, size=1 if act_quant == W.ACT_PER_TENSOR else m_cap)).astype(np.float32)
    sb = np.ldexp(1.0, g.integers(-2, 3, size=E if w_quant == W.W_PER_EXPERT else E * N)).astype(np.float32)
    print(f"mxfp4 exact act={act_quant} w={w_quant} K={K}", flush=True)
    ref = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    M = int(seg[-1])
    assert np.array_equal(c[:M], ref[:M])


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL)])
@pytest.mark.parametrize("dims", [((37, 0, 300, 5, 129), 256, 512), ((1,), 128, 128),
                                  ((17, 40), 48, 256), ((0, 260, 3), 400, 1024)])
def test_mxfp4_gemm_random(act_quant, w_quant, dims):
    counts, N, K = dims
    g = np.random.default_rng(5)
    seg = _seg(counts)
    E = len(counts)
    m_cap = int(seg[-1]) + 7
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (m_cap, K))]
    b_fp4, b_e8m0 = _fp4_weights(g, E, N, K)
    sa = g.uniform(1e-3, 4e-3, 1 if act_quant == W.ACT_PER_TENSOR else m_cap).astype(np.float32)
    sb = g.uniform(0.5, 2.0, E if w_quant == W.W_PER_EXPERT else E * N).astype(np.float32)
    print(f"mxfp4 random counts={counts} N={N} K={K} act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    M = int(seg[-1])
    if M == 0:
        return
    rows = np.arange(M)
    worst = G.assert_sum_close(c[:M], ref[:M], abs_products_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb,
                                                                 w_quant, seg, rows), K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")


# Row capacity of at most 64 rows per local expert with K a multiple of 256 and
# at least 1024: the weight-streaming kernel (units of 8 rows x 16 columns over
# 256-deep K steps). Segments of 1-8 rows (one unit high), 9, 17 and 24 (two and
# three units sharing the expert's weights), empty experts, and column counts
# that are not a multiple of 64.
STREAM_COUNTS = (3, 0, 17, 9, 1, 8, 0, 24, 5, 2)


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL),
                                               (W.ACT_PER_TOKEN, W.W_PER_EXPERT)])
def test_mxfp4_gemm_exact_case_streaming(act_quant, w_quant):
    """The exact case of test_mxfp4_gemm_exact_case on the weight-streaming path;
    bit-identical."""
    g = np.random.default_rng(13)
    seg = _seg(STREAM_COUNTS)
    E, K, N = len(STREAM_COUNTS), 1024, 80
    m_cap = 64 * E
    a_q = W.to_e4m3_codes(g.integers(-1, 2, size=(m_cap, K)).astype(np.float32))
    nib = np.array([0, 1, 2, 4, 9, 10, 12], np.uint8)[g.integers(0, 7, size=(E, N, K))]
    b_fp4 = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    b_e8m0 = g.integers(126, 128, size=(E, N, K // 32)).astype(np.uint8)
    sa = np.ldexp(1.0, g.integers(-2, 3, size=1 if act_quant == W.ACT_PER_TENSOR else m_cap)).astype(np.float32)
    sb = np.ldexp(1.0, g.integers(-2, 3, size=E if w_quant == W.W_PER_EXPERT else E * N)).astype(np.float32)
    print(f"mxfp4 exact streaming act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    M = int(seg[-1])
    assert np.array_equal(c[:M], ref[:M])


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL)])
@pytest.mark.parametrize("N,K", [(272, 2048), (80, 1024), (1040, 7168), (96, 3584), (64, 2560)])
def test_mxfp4_gemm_random_streaming(act_quant, w_quant, N, K):
    """Random codes and block scales on the weight-streaming path (K = 2560, whose
    last group of eight 256-deep steps would have two, takes the tiled kernel):
    within one bf16 step plus both sides' summation bounds."""
    g = np.random.default_rng(17)
    seg = _seg(STREAM_COUNTS)
    E = len(STREAM_COUNTS)
    m_cap = 64 * E
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (m_cap, K))]
    b_fp4, b_e8m0 = _fp4_weights(g, E, N, K)
    sa = g.uniform(1e-3, 4e-3, 1 if act_quant == W.ACT_PER_TENSOR else m_cap).astype(np.float32)
    sb = g.uniform(0.5, 2.0, E if w_quant == W.W_PER_EXPERT else E * N).astype(np.float32)
    print(f"mxfp4 random streaming N={N} K={K} act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    M = int(seg[-1])
    rows = np.arange(M)
    worst = G.assert_sum_close(c[:M], ref[:M], abs_products_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb,
                                                                 w_quant, seg, rows), K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")


# One case per FP4 GEMM kernel the library picks: (modes, local experts, m_cap, N, K).
FP4_PATHS = {
    "streaming": (W.ACT_PER_TENSOR, W.W_PER_EXPERT, 10, 320, 80, 1024),  # at most 64 rows per expert
    "tiles256k": (W.ACT_PER_TOKEN, W.W_PER_CHANNEL, 3, 300, 256, 512),   # 256-deep K steps
    "tiles128k": (W.ACT_PER_TOKEN, W.W_PER_EXPERT, 3, 300, 256, 384),    # K not a multiple of 256
}


def _fp4_case(seed, path):
    act_quant, w_quant, E, m_cap, N, K = FP4_PATHS[path]
    g = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (m_cap, K))]
    b_fp4, b_e8m0 = _fp4_weights(g, E, N, K)
    sa = g.uniform(1e-3, 4e-3, 1 if act_quant == W.ACT_PER_TENSOR else m_cap).astype(np.float32)
    sb = g.uniform(0.5, 2.0, E if w_quant == W.W_PER_EXPERT else E * N).astype(np.float32)
    return act_quant, w_quant, a_q, sa, b_fp4, b_e8m0, sb


@pytest.mark.parametrize("path", list(FP4_PATHS))
def test_mxfp4_gemm_all_segments_empty(path):
    """Every segment empty (M = 0): no row of C is written."""
    act_quant, w_quant, a_q, sa, b_fp4, b_e8m0, sb = _fp4_case(3, path)
    seg = np.zeros(b_fp4.shape[0] + 1, np.int32)
    print(f"mxfp4 all empty {path} m_cap={a_q.shape[0]} N={b_fp4.shape[1]} K={a_q.shape[1]}", flush=True)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    assert np.isnan(G.bf16_to_f64(c)).all(), "a row of C was written although every segment is empty"


@pytest.mark.parametrize("path", list(FP4_PATHS))
def test_mxfp4_gemm_seg_clamped(path):
    """seg_indptr values outside [0, m_cap] are clamped before use; compared with
    the oracle on the clamped offsets (every row of C is then written)."""
    act_quant, w_quant, a_q, sa, b_fp4, b_e8m0, sb = _fp4_case(4, path)
    E, m_cap, K = b_fp4.shape[0], a_q.shape[0], a_q.shape[1]
    seg = np.array([-5] + [7] * (E - 1) + [m_cap + 50], np.int32)
    seg_c = np.clip(seg, 0, m_cap).astype(np.int32)
    print(f"mxfp4 clamped seg {path} seg={seg.tolist()}", flush=True)
    ref = oracle.grouped_gemm_mxfp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg_c)
    c = G.run_gemm_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg)
    # random codes cancel in places, so the bound is the summation error of both
    # sides (as in the other random-code cases), not a relative tolerance
    worst = G.assert_sum_close(c, ref, abs_products_fp4(a_q, sa, act_quant, b_fp4, b_e8m0, sb, w_quant, seg_c,
                                                        np.arange(m_cap)), K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")


@pytest.mark.parametrize("name,which", [("dsv3_prefill_ep_fp4", "w13"), ("dsv3_prefill_ep_fp4", "w2"),
                                        ("dsv3_decode_ep_fp4", "w13"), ("dsv3_decode_ep_fp4", "w2")])
def test_mxfp4_gemm_full_size_sampled_rows(name, which):
    cfg = W.CONFIGS[name]
    inp = W.gen_layer_inputs(cfg, weights=False)
    ids, _ = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                   cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    s2d, d2s, seg = oracle.permute(ids, cfg.expert_start, cfg.num_local, cfg.m_cap)
    M = int(seg[-1])
    g = np.random.default_rng(1)
    if which == "w13":
        K, N = cfg.H, 2 * cfg.I
        a_q, sa = oracle.pre_reorder_quant(inp.x, s2d, cfg.topk, cfg.act_quant, cfg.m_cap)
    else:
        K, N = cfg.I, cfg.H
        a_q = (g.integers(0, 0x7E, (cfg.m_cap, K)) | (g.integers(0, 2, (cfg.m_cap, K)) * 0x80)).astype(np.uint8)
        sa = g.uniform(1e-3, 4e-3, cfg.m_cap).astype(np.float32)
    b_fp4, b_e8m0, sb = W.gen_weights_fp4(cfg, which)
    print(f"mxfp4 full {name} {which} M={M} N={N} K={K}", flush=True)
    c = G.run_gemm_fp4(a_q, sa, cfg.act_quant, b_fp4, b_e8m0, sb, cfg.w_quant, seg)
    # random rows plus every non-empty segment's first and last row
    nonempty = np.nonzero(np.diff(seg) > 0)[0]
    edges = np.concatenate([seg[nonempty], seg[nonempty + 1] - 1])
    rows = np.unique(np.concatenate([g.integers(0, M, 44), [0, M - 1], edges]))
    rows = rows[rows < M]
    ref = oracle.grouped_gemm_mxfp4_rows(a_q, sa, cfg.act_quant, b_fp4, b_e8m0, sb, cfg.w_quant, seg, rows)
    G.assert_close_layer(c[rows], ref, what="C rows")
    worst = G.assert_sum_close(c[rows], ref, abs_products_fp4(a_q, sa, cfg.act_quant, b_fp4, b_e8m0, sb,
                                                               cfg.w_quant, seg, rows), K, what="C rows")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")
