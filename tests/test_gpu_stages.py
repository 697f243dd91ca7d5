"""Stage-isolated GPU parity: each libmoe stage against the CPU oracle on the
same seeded inputs, through the C ABI.

Bit-exact: expert ids, src2dst / dst2src / seg_indptr, FP8 codes and scales.
Within tolerance: routing weights (4e-6 relative), GEMM outputs (the layer
tolerance, atol 1e-2 + rtol 2e-2, and exact in the exact-arithmetic case),
combine (one bf16 ulp of the fp64 sum).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

FULL = ["tiny", "dsv3_decode_ep", "dsv3_prefill_ep", "mixtral", "skewed_block"]


@functools.lru_cache(maxsize=2)
def routed(name, seed=0):
    """Token bits, logits/bias and the oracle's routing for a named workload."""
    cfg = W.CONFIGS[name]
    inp = W.gen_layer_inputs(cfg, seed=seed, weights=False)
    ids, w = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                   cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    return cfg, inp, ids, w


def check_weights(w, ref):
    assert np.all(np.abs(w.astype(np.float64) - ref) <= 4e-6 * np.abs(ref) + 1e-12)


# ---- stage 1 ------------------------------------------------------------------------

@pytest.mark.parametrize("name", FULL)
def test_select_experts_workloads(name):
    cfg, inp, ids_ref, w_ref = routed(name)
    print(f"select_experts {name} T={cfg.T} E={cfg.E}", flush=True)
    ids, w = G.run_select(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                          cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    assert np.array_equal(ids, ids_ref)
    check_weights(w, w_ref)


@pytest.mark.parametrize("case", ["ties_softmax", "ties_sigmoid_grouped", "k_eq_e", "no_renorm",
                                  "no_rsf", "odd_T", "E512", "one_token"])
def test_select_experts_edges(case):
    g = np.random.default_rng(11)
    kw = dict(topk=2, n_group=1, topk_group=1, score_fn=W.SCORE_SOFTMAX, renormalize=1, rsf=1.0,
              apply_rsf=1)
    bias = None
    if case == "ties_softmax":
        logits = g.integers(-2, 3, (37, 16)).astype(np.float32)
        kw.update(topk=5)
    elif case == "ties_sigmoid_grouped":
        logits = g.integers(-1, 2, (37, 64)).astype(np.float32)
        bias = np.zeros(64, np.float32)
        kw.update(topk=6, n_group=8, topk_group=3, score_fn=W.SCORE_SIGMOID, rsf=2.5)
    elif case == "k_eq_e":
        logits = g.standard_normal((33, 8)).astype(np.float32)
        kw.update(topk=8)
    elif case == "no_renorm":
        logits = g.standard_normal((40, 128)).astype(np.float32)
        kw.update(topk=8, renormalize=0)
    elif case == "no_rsf":
        logits = g.standard_normal((40, 256)).astype(np.float32) * 2
        bias = (g.standard_normal(256) * 0.01).astype(np.float32)
        kw.update(topk=8, n_group=8, topk_group=4, score_fn=W.SCORE_SIGMOID, rsf=2.5, apply_rsf=0)
    elif case == "odd_T":
        logits = g.standard_normal((5, 256)).astype(np.float32)
        bias = (g.standard_normal(256) * 0.01).astype(np.float32)
        kw.update(topk=8, n_group=8, topk_group=4, score_fn=W.SCORE_SIGMOID, rsf=2.5)
    elif case == "E512":
        logits = g.standard_normal((9, 512)).astype(np.float32)
        kw.update(topk=32)
    else:
        logits = g.standard_normal((1, 32)).astype(np.float32)
        bias = (g.standard_normal(32) * 0.1).astype(np.float32)
        kw.update(topk=4, n_group=4, topk_group=2, score_fn=W.SCORE_SIGMOID, renormalize=0)
    print(f"select_experts edge {case}", flush=True)
    ids_ref, w_ref = oracle.select_experts(logits, bias, kw["topk"], kw["n_group"], kw["topk_group"],
                                           kw["score_fn"], kw["renormalize"], kw["rsf"], kw["apply_rsf"])
    ids, w = G.run_select(logits, bias, **kw)
    assert np.array_equal(ids, ids_ref)
    check_weights(w, w_ref)


@pytest.mark.parametrize("case", [
    # (E, topk, n_group, topk_group, score_fn, T): sixteen lanes per token, a group
    # spanning 1, 2, 4, 8 or 16 lanes, up to 16 output slots, partial blocks
    (256, 8, 16, 8, W.SCORE_SIGMOID, 33),
    (256, 8, 8, 4, W.SCORE_SIGMOID, 17),
    (128, 6, 4, 2, W.SCORE_SIGMOID, 40),
    (256, 16, 2, 1, W.SCORE_SIGMOID, 21),
    (64, 16, 1, 1, W.SCORE_SIGMOID, 19),
    (64, 16, 1, 1, W.SCORE_SOFTMAX, 50),
    (128, 1, 1, 1, W.SCORE_SOFTMAX, 3),
    (256, 12, 1, 1, W.SCORE_SOFTMAX, 16),
])
def test_select_experts_row_layout(case):
    E, topk, n_group, topk_group, score_fn, T = case
    g = np.random.default_rng(E * 31 + topk)
    logits = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    logits[::5, :: 3] = np.round(logits[::5, ::3])  # some exact ties
    bias = (g.standard_normal(E) * 0.01).astype(np.float32) if score_fn == W.SCORE_SIGMOID else None
    kw = dict(topk=topk, n_group=n_group, topk_group=topk_group, score_fn=score_fn, renormalize=1,
              rsf=2.5, apply_rsf=1)
    print(f"select_experts row layout {case}", flush=True)
    ids_ref, w_ref = oracle.select_experts(logits, bias, topk, n_group, topk_group, score_fn, 1, 2.5, 1)
    ids, w = G.run_select(logits, bias, **kw)
    assert np.array_equal(ids, ids_ref)
    check_weights(w, w_ref)


def test_select_experts_unaligned_bias():
    """A correction bias that is not 16-byte aligned takes the one-wave-per-token
    kernel; results are the same."""
    g = np.random.default_rng(3)
    T, E = 24, 256
    logits = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    bias = (g.standard_normal(E) * 0.01).astype(np.float32)
    ids_ref, w_ref = oracle.select_experts(logits, bias, 8, 8, 4, W.SCORE_SIGMOID, 1, 2.5, 1)
    store = G.up(np.concatenate([[0.0], bias]).astype(np.float32))
    bt = store[1:]
    ids = G.Guarded((T, 8), torch.int32)
    w = G.Guarded((T, 8), torch.float32)
    G.moe.moe_select_experts(G.up(logits), bt, ids.t, w.t, topk=8, n_group=8, topk_group=4,
                             score_fn=W.SCORE_SIGMOID, renormalize=1, routed_scaling_factor=2.5,
                             apply_rsf=1)
    torch.cuda.synchronize()
    ids.check("topk_ids")
    w.check("topk_weights")
    assert np.array_equal(ids.t.cpu().numpy(), ids_ref)
    check_weights(w.t.cpu().numpy(), w_ref)


# ---- stage 2 ----------------------------------------------------------------------

def check_pre(res, ref_perm, ref_q, act_quant, H):
    s2d, d2s, seg = ref_perm
    a_q_ref, a_s_ref = ref_q
    assert np.array_equal(res["seg"], seg)
    assert np.array_equal(res["src2dst"], s2d)
    assert np.array_equal(res["dst2src"], d2s)
    M = int(seg[-1])
    assert np.array_equal(res["a_q"][:M], a_q_ref[:M])
    if act_quant == W.ACT_PER_TENSOR:
        assert res["a_scale"][0].view(np.uint32) == a_s_ref[0].view(np.uint32)
    else:
        Gq = 1 if act_quant == W.ACT_PER_TOKEN else -(-H // 128)
        assert np.array_equal(res["a_scale"][:M * Gq].view(np.uint32), a_s_ref[:M * Gq].view(np.uint32))


def pre_case(x_bits, ids, expert_start, num_local, act_quant):
    T, H = x_bits.shape
    topk = ids.shape[1]
    m_cap = T * min(topk, num_local)
    ref_perm = oracle.permute(ids, expert_start, num_local, m_cap)
    ref_q = oracle.pre_reorder_quant(x_bits, ref_perm[0], topk, act_quant, m_cap)
    res = G.run_pre(x_bits, ids, expert_start, num_local, act_quant)
    check_pre(res, ref_perm, ref_q, act_quant, H)


@pytest.mark.parametrize("name", FULL)
def test_pre_reorder_workloads(name):
    cfg, inp, ids, _ = routed(name)
    print(f"pre_reorder {name} T={cfg.T} H={cfg.H}", flush=True)
    pre_case(inp.x, ids, cfg.expert_start, cfg.num_local, cfg.act_quant)


@pytest.mark.parametrize("act_quant", [W.ACT_PER_TENSOR, W.ACT_PER_TOKEN, W.ACT_PER_GROUP])
# (T, H, E, topk, expert_start, num_local). The library derives the permutation in
# one launch for up to 2048 pairs with at most 4096 expert x chunk entries, in a
# single count-and-scan block up to 4096 pairs, and in separate count and scan
# passes beyond: the last four shapes sit at and past those limits.
@pytest.mark.parametrize("shape", [(1, 16, 4, 2, 0, 8), (63, 144, 16, 4, 3, 5), (65, 9216, 8, 8, 0, 8),
                                   (200, 256, 64, 6, 10, 20), (130, 384, 8, 2, 0, 1),
                                   (256, 128, 256, 8, 0, 128), (256, 64, 256, 8, 0, 200),
                                   (500, 256, 64, 8, 0, 64), (700, 64, 16, 6, 0, 16)])
def test_pre_reorder_ragged(act_quant, shape):
    T, H, E, topk, start, nl = shape
    g = np.random.default_rng(T * 7 + H)
    x = g.standard_normal((T, H)).astype(np.float32) * (2.0 ** (np.arange(T) % 9 - 4))[:, None]
    x[T // 2] = 0.0
    ids = np.stack([g.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    print(f"pre_reorder ragged T={T} H={H} E={E} k={topk} local=[{start},{start + nl}) mode={act_quant}",
          flush=True)
    pre_case(W.to_bf16_bits(x.astype(np.float32)), ids, start, nl, act_quant)


def test_pre_reorder_no_local_and_empty():
    g = np.random.default_rng(3)
    x = W.to_bf16_bits(g.standard_normal((40, 64)).astype(np.float32))
    ids = np.stack([g.permutation(16)[:4] for _ in range(40)]).astype(np.int32)
    print("pre_reorder no local experts", flush=True)
    res = G.run_pre(x, ids, 16, 4, W.ACT_PER_TOKEN)       # experts 16..19 do not occur
    assert np.all(res["seg"] == 0) and np.all(res["src2dst"] == -1) and np.all(res["dst2src"] == -1)
    print("pre_reorder zero local experts", flush=True)
    res = G.run_pre(x, ids, 0, 0, W.ACT_PER_TOKEN)
    assert np.all(res["seg"] == 0) and np.all(res["src2dst"] == -1)


def test_e4m3_encoder_on_device_matches_oracle():
    """Rows whose |max| is 448 have scale 1: the codes are the e4m3 rounding of the
    bf16 values themselves, covering every e4m3 midpoint and its bf16 neighbours."""
    table = oracle.e4m3_decode_table().astype(np.float64)
    pos = table[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = []
    for m in mids:
        b = int(W.to_bf16_bits(np.array([m], np.float32))[0])
        vals += [b - 1, b, b + 1]
    vals = np.array(vals, dtype=np.uint16)
    vals = np.concatenate([vals, vals | 0x8000, W.to_bf16_bits(pos.astype(np.float32)),
                           np.array([0x0000, 0x8000, 0x0001, 0x8001], np.uint16)])
    H = 256
    n = -(-len(vals) // (H - 1))
    rows = np.zeros((n, H), dtype=np.uint16)
    flat = np.zeros(n * (H - 1), dtype=np.uint16)
    flat[:len(vals)] = vals
    rows[:, :H - 1] = flat.reshape(n, H - 1)
    rows[:, H - 1] = W.to_bf16_bits(np.array([448.0], np.float32))[0]
    ids = np.zeros((n, 1), np.int32)
    print(f"e4m3 encoder rows={n}", flush=True)
    res = G.run_pre(rows, ids, 0, 1, W.ACT_PER_TOKEN)
    assert np.all(res["a_scale"][:n] == 1.0)
    expect = np.array([[oracle.e4m3_encode(float(v)) for v in W.bf16_bits_to_f32(r)] for r in rows],
                      dtype=np.uint8)
    assert np.array_equal(res["a_q"][:n], expect)


# ---- stage 3 ------------------------------------------------------------------------

from tests.test_oracle_layer import _exact_gemm_case  # noqa: E402


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL),
                                               (W.ACT_PER_GROUP, W.W_BLOCK),
                                               (W.ACT_PER_GROUP, W.W_PER_CHANNEL),
                                               (W.ACT_PER_TOKEN, W.W_BLOCK)])
def test_grouped_gemm_exact_case(act_quant, w_quant):
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant)
    print(f"grouped_gemm exact act={act_quant} w={w_quant}", flush=True)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    assert np.array_equal(c[:M], expect[:M])


# Cases with m_cap at least 128 rows per local expert, where the library takes
# the 256 x 256 tile kernel for the block-scaled modes (the others keep the
# 128 x 256 one): segments of every size around the 8-row DMA instructions, the
# 16-row MFMA blocks and the 128- and 256-row tiles (empty ones too), and column
# counts that leave a partial column tile.
BIG_COUNTS = (1, 15, 16, 17, 0, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300)
ALL_MODES = [(W.ACT_PER_TENSOR, W.W_PER_EXPERT), (W.ACT_PER_TOKEN, W.W_PER_EXPERT),
             (W.ACT_PER_TOKEN, W.W_PER_CHANNEL), (W.ACT_PER_GROUP, W.W_BLOCK),
             (W.ACT_PER_GROUP, W.W_PER_CHANNEL), (W.ACT_PER_TOKEN, W.W_BLOCK)]


@pytest.mark.parametrize("act_quant,w_quant", ALL_MODES)
def test_grouped_gemm_exact_case_256_tiles(act_quant, w_quant):
    """The exact-arithmetic case with m_cap at least 128 rows per expert (the
    256 x 256 tile kernel in the block-scaled modes): segments longer than a
    tile, one row, one full tile, and a partial column tile; bit-exact."""
    counts, N = (300, 0, 17, 256, 1), 384
    m_cap_min = 128 * len(counts)
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant, counts=counts, N=N,
                                                            extra=m_cap_min - sum(counts) + 9)
    assert m_cap >= m_cap_min
    print(f"grouped_gemm exact 256-row tiles act={act_quant} w={w_quant}", flush=True)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    assert np.array_equal(c[:M], expect[:M])


@pytest.mark.parametrize("act_quant,w_quant", ALL_MODES)
@pytest.mark.parametrize("N,K", [(256, 256), (384, 512), (160, 128)])
def test_grouped_gemm_random_256_tiles(act_quant, w_quant, N, K):
    """Random finite codes with m_cap at least 128 rows per expert (the 256 x 256
    tile kernel in the block-scaled modes), every segment size around the row
    boundaries: within one bf16 step plus both sides' summation bounds."""
    if w_quant == W.W_BLOCK and N % 128:
        N = 128 * -(-N // 128)
    extra = 128 * len(BIG_COUNTS) - sum(BIG_COUNTS) + 13
    a_q, sa, b_q, sb, seg = _rand_gemm(9, BIG_COUNTS, N, K, act_quant, w_quant, extra=extra)
    assert a_q.shape[0] >= 128 * len(BIG_COUNTS)
    print(f"grouped_gemm random 256-row tiles N={N} K={K} act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    G.assert_close_layer(c[:M], ref[:M], what="C")
    rows = np.arange(M)
    worst = G.assert_sum_close(c[:M], ref[:M], abs_products(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows),
                               K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")


# Cases with m_cap at most 64 rows per local expert, K a multiple of 1024 and no
# K-dependent scale, where the library streams each expert's weights once (one
# wave per unit of 16 rows x 16 columns of an expert): one-unit-high segments
# (1, 2, 3, 5, 16 rows), two- and three-unit ones (17, 33, 48), whose weights
# the units share through L2, empty experts, and column counts that are not a
# multiple of 64.
SMALL_COUNTS = (3, 0, 17, 33, 1, 16, 0, 48, 5, 2)
PLAIN_MODES = [(W.ACT_PER_TENSOR, W.W_PER_EXPERT), (W.ACT_PER_TOKEN, W.W_PER_EXPERT),
               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL), (W.ACT_PER_TENSOR, W.W_PER_CHANNEL)]


@pytest.mark.parametrize("act_quant,w_quant", PLAIN_MODES)
def test_grouped_gemm_exact_case_streaming(act_quant, w_quant):
    """The exact-arithmetic case on the weight-streaming path; bit-exact."""
    counts, N, K = SMALL_COUNTS, 80, 1024
    m_cap_max = 32 * len(counts)
    a_q, sa, b_q, sb, seg, expect, m_cap = _exact_gemm_case(act_quant, w_quant, counts=counts, N=N, K=K,
                                                            extra=m_cap_max - sum(counts))
    assert m_cap <= m_cap_max
    print(f"grouped_gemm exact streaming act={act_quant} w={w_quant}", flush=True)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    assert np.array_equal(c[:M], expect[:M])


@pytest.mark.parametrize("act_quant,w_quant", PLAIN_MODES)
@pytest.mark.parametrize("N,K", [(272, 2048), (64, 1024), (1040, 3072)])
def test_grouped_gemm_random_streaming(act_quant, w_quant, N, K):
    """Random finite codes on the weight-streaming path: within one bf16 step
    plus both sides' summation bounds."""
    extra = 32 * len(SMALL_COUNTS) - sum(SMALL_COUNTS)
    a_q, sa, b_q, sb, seg = _rand_gemm(11, SMALL_COUNTS, N, K, act_quant, w_quant, extra=extra)
    assert a_q.shape[0] <= 32 * len(SMALL_COUNTS)
    print(f"grouped_gemm random streaming N={N} K={K} act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    G.assert_close_layer(c[:M], ref[:M], what="C")
    rows = np.arange(M)
    worst = G.assert_sum_close(c[:M], ref[:M], abs_products(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows),
                               K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g}")


def _rand_gemm(seed, counts, N, K, act_quant, w_quant, extra=7):
    g = np.random.default_rng(seed)
    counts = np.asarray(counts)
    E_l = len(counts)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m_cap = int(seg[-1]) + extra
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a_q = finite[g.integers(0, len(finite), (m_cap, K))]
    b_q = finite[g.integers(0, len(finite), (E_l, N, K))]
    na = W.a_scale_numel(act_quant, m_cap, K)
    nb = W.b_scale_numel(w_quant, E_l, N, K)
    sa = g.uniform(1e-3, 4e-3, na).astype(np.float32)
    sb = g.uniform(1e-4, 4e-4, nb).astype(np.float32)
    return a_q, sa, b_q, sb, seg


def abs_products(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows):
    """sum_k |a_hat[r,k] * b_hat[e,n,k]| for the given rows (fp64), the scale of the
    fp32 summation error of either side. Each expert's |b_hat| is formed once."""
    table = np.abs(oracle.e4m3_decode_table().astype(np.float64))
    sa = np.asarray(sa).reshape(-1)
    sb = np.asarray(sb).reshape(-1)
    m_cap, K = a_q.shape
    E_l, N, _ = b_q.shape
    KB, NB = -(-K // 128), -(-N // 128)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), N))
    experts = np.searchsorted(seg, rows, side="right") - 1
    for e in np.unique(experts):
        idx = np.nonzero(experts == e)[0]
        a = np.empty((len(idx), K))
        for q, i in enumerate(idx):
            r = int(rows[i])
            if act_quant == W.ACT_PER_TENSOR:
                sa_row = np.full(K, sa[0], np.float64)
            elif act_quant == W.ACT_PER_TOKEN:
                sa_row = np.full(K, sa[r], np.float64)
            else:
                sa_row = np.repeat(sa[r * KB:(r + 1) * KB].astype(np.float64), 128)[:K]
            a[q] = table[a_q[r]] * np.abs(sa_row)
        bt = table[b_q[e]]
        if w_quant == W.W_PER_EXPERT:
            bt = bt * abs(float(sb[e]))
        elif w_quant == W.W_PER_CHANNEL:
            bt = bt * np.abs(sb[e * N:(e + 1) * N].astype(np.float64))[:, None]
        else:
            blk = np.abs(sb[e * NB * KB:(e + 1) * NB * KB].astype(np.float64)).reshape(NB, KB)
            bt = bt * np.repeat(np.repeat(blk, 128, 0), 128, 1)[:N, :K]
        out[idx] = a @ bt.T
        del bt
    return out


@pytest.mark.parametrize("act_quant,w_quant", [(W.ACT_PER_TENSOR, W.W_PER_EXPERT),
                                               (W.ACT_PER_TOKEN, W.W_PER_CHANNEL),
                                               (W.ACT_PER_GROUP, W.W_BLOCK)])
@pytest.mark.parametrize("dims", [((37, 0, 300, 5, 129), 256, 512), ((1,), 128, 128),
                                  ((17, 40), 48, 80), ((0, 260, 3), 384, 1024)])
def test_grouped_gemm_random(act_quant, w_quant, dims):
    counts, N, K = dims
    if w_quant == W.W_BLOCK and (N % 128 or K % 128):
        N, K = 128 * -(-N // 128), 128 * -(-K // 128)
    a_q, sa, b_q, sb, seg = _rand_gemm(5, counts, N, K, act_quant, w_quant)
    print(f"grouped_gemm random counts={counts} N={N} K={K} act={act_quant} w={w_quant}", flush=True)
    ref = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    M = seg[-1]
    G.assert_close_layer(c[:M], ref[:M], what="C")
    rows = np.arange(M)
    worst = G.assert_sum_close(c[:M], ref[:M], abs_products(a_q, sa, act_quant, b_q, sb, w_quant, seg, rows),
                               K, what="C")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g} (2^{np.log2(max(worst, 1e-30)):.1f})")


@pytest.mark.parametrize("name,which", [("dsv3_prefill_ep", "w13"), ("dsv3_prefill_ep", "w2"),
                                        ("mixtral", "w13"), ("mixtral", "w2"),
                                        ("skewed_block", "w13"), ("skewed_block", "w2"),
                                        ("dsv3_decode_ep", "w13"), ("dsv3_decode_ep", "w2")])
def test_grouped_gemm_full_size_sampled_rows(name, which):
    """Full workload shapes in the benchmark's launch configuration. Sampled rows
    (all N columns) are recomputed by the oracle one row at a time: 44 random
    rows, the first and last row, and the first and last row of every non-empty
    expert segment (where a tile-table or row-scale indexing error would show).
    The Mixtral w2 case is the longest K loop (K = 14336) with the per-tensor
    activation scale."""
    cfg, inp, ids, _ = routed(name)
    m_cap = cfg.m_cap
    s2d, d2s, seg = oracle.permute(ids, cfg.expert_start, cfg.num_local, m_cap)
    M = int(seg[-1])
    g = np.random.default_rng(1)
    if which == "w13":
        K, N = cfg.H, 2 * cfg.I
        a_q, sa = oracle.pre_reorder_quant(inp.x, s2d, cfg.topk, cfg.act_quant, m_cap)
    else:
        K, N = cfg.I, cfg.H
        a_q = g.integers(0, 0x7E, (m_cap, K)).astype(np.uint8) | (g.integers(0, 2, (m_cap, K)) * 0x80).astype(np.uint8)
        sa = g.uniform(1e-3, 4e-3, W.a_scale_numel(cfg.act_quant, m_cap, K)).astype(np.float32)
    full = G.layer_inputs(name)
    b_q, sb = (full.w13, full.w13_scale) if which == "w13" else (full.w2, full.w2_scale)
    print(f"grouped_gemm full {name} {which} M={M} N={N} K={K}", flush=True)
    c = G.run_gemm(a_q, sa, cfg.act_quant, b_q, sb, cfg.w_quant, seg)
    nonempty = np.nonzero(seg[1:] > seg[:-1])[0]
    edges = np.concatenate([seg[nonempty], seg[nonempty + 1] - 1])
    rows = np.unique(np.concatenate([g.integers(0, M, 44), [0, M - 1], edges]))
    rows = rows[rows < M]
    ref = oracle.grouped_gemm_rows(a_q, sa, cfg.act_quant, b_q, sb, cfg.w_quant, seg, rows)
    G.assert_close_layer(c[rows], ref, what="C rows")
    worst = G.assert_sum_close(c[rows], ref, abs_products(a_q, sa, cfg.act_quant, b_q, sb, cfg.w_quant,
                                                          seg, rows), K, what="C rows")
    print(f"worst |diff| beyond one ulp, relative to sum|products|: {worst:.3g} (2^{np.log2(max(worst, 1e-30)):.1f})")


# One case per GEMM kernel the library picks: (modes, local experts, m_cap, N, K).
GEMM_PATHS = {
    # no K-dependent scale, K/128 >= 4, at most 64 rows per expert: weight streaming
    "streaming": (W.ACT_PER_TENSOR, W.W_PER_EXPERT, 10, 320, 80, 1024),
    # K-dependent scales, at least 128 rows per expert: 256 x 256 tiles
    "tiles256": (W.ACT_PER_GROUP, W.W_BLOCK, 3, 404, 256, 512),
    # 128 x 256 tiles, without and with K-dependent scales
    "tiles128": (W.ACT_PER_TOKEN, W.W_PER_CHANNEL, 4, 400, 256, 512),
    "tiles128_kdep": (W.ACT_PER_TOKEN, W.W_BLOCK, 4, 400, 256, 512),
    # K not a multiple of 128: the plain tiled kernel
    "plain": (W.ACT_PER_TOKEN, W.W_PER_EXPERT, 3, 150, 48, 80),
}


@pytest.mark.parametrize("path", list(GEMM_PATHS))
def test_grouped_gemm_all_segments_empty(path):
    """Every segment empty (M = 0, seg_indptr all zeros) with m_cap rows of
    codes present: no tile exists and no row of C is written."""
    act_quant, w_quant, E_l, m_cap, N, K = GEMM_PATHS[path]
    a_q, sa, b_q, sb, _ = _rand_gemm(17, [m_cap] + [0] * (E_l - 1), N, K, act_quant, w_quant, extra=0)
    seg = np.zeros(E_l + 1, np.int32)
    print(f"grouped_gemm all empty {path} E_l={E_l} m_cap={m_cap} N={N} K={K}", flush=True)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    assert np.isnan(G.bf16_to_f64(c)).all(), "a row of C was written although every segment is empty"


@pytest.mark.parametrize("path", list(GEMM_PATHS))
def test_grouped_gemm_seg_clamped(path):
    """seg_indptr values outside [0, m_cap] are clamped before use: a negative
    start reads as 0 and a last end past m_cap as m_cap, so the last expert owns
    every row from its start to m_cap. Compared with the oracle on the clamped
    offsets."""
    act_quant, w_quant, E_l, m_cap, N, K = GEMM_PATHS[path]
    a_q, sa, b_q, sb, _ = _rand_gemm(23, [m_cap] + [0] * (E_l - 1), N, K, act_quant, w_quant, extra=0)
    mid = 7 if E_l > 2 else m_cap // 3
    seg = np.array([-5] + [mid] * (E_l - 1) + [m_cap + 50], np.int32)
    seg_c = np.clip(seg, 0, m_cap).astype(np.int32)
    print(f"grouped_gemm clamped seg {path} seg={seg.tolist()}", flush=True)
    ref = oracle.grouped_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg_c)
    c = G.run_gemm(a_q, sa, act_quant, b_q, sb, w_quant, seg)
    G.assert_close_layer(c, ref, what="C")
    G.assert_sum_close(c, ref, abs_products(a_q, sa, act_quant, b_q, sb, w_quant, seg_c, np.arange(m_cap)),
                       K, what="C")


# ---- stage 4 ------------------------------------------------------------------------

@pytest.mark.parametrize("act_quant", [W.ACT_PER_TENSOR, W.ACT_PER_TOKEN, W.ACT_PER_GROUP])
# In the per-group mode, I / 16 not a multiple of 64 (768, 384, 1152) takes the
# kernel that packs 16-column chunks of several rows into each wave.
@pytest.mark.parametrize("dims", [((20, 0, 31), 64), ((300, 17), 2048), ((5,), 9216), ((64, 64), 768),
                                  ((7, 3), 3072), ((9,), 5120), ((13, 0, 6), 384), ((1, 40, 2), 1152)])
def test_act_requant_ragged(act_quant, dims):
    counts, I = dims
    g = np.random.default_rng(len(counts) * 100 + I)
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m_cap = int(seg[-1]) + 9
    gu = W.to_bf16_bits((g.standard_normal((m_cap, 2 * I)) * 1.7).astype(np.float32))
    print(f"act_requant counts={counts} I={I} mode={act_quant}", flush=True)
    a_ref, s_ref = oracle.act_requant(gu, seg, act_quant)
    a_q, a_s = G.run_act(gu, seg, act_quant)
    M = int(seg[-1])
    assert np.array_equal(a_q[:M], a_ref[:M])
    Gq = 1 if act_quant == W.ACT_PER_TOKEN else -(-I // 128)
    n = 1 if act_quant == W.ACT_PER_TENSOR else M * Gq
    assert np.array_equal(a_s[:n].view(np.uint32), s_ref[:n].view(np.uint32))


def _act_edge_rows(I=256, seed=5):
    """gate / up rows with extreme values: signed zeros, bf16 subnormals, values
    around 2^-103 (where the kernel's division skips its range scaling), huge
    gates whose exp(-g) clamps, and rows whose amax falls below the 1e-10 floor."""
    g = np.random.default_rng(seed)
    special = np.array([0.0, -0.0, 1e-38, -1e-38, 2.0 ** -103, -(2.0 ** -103), 2.0 ** -102, -(2.0 ** -104),
                        1e-35, -1e-35, 1e-20, -1e-20, 80.0, -80.0, 80.5, -80.5, 100.0, -100.0, 1e4, -1e4,
                        1e30, -1e30, 1e35, -1e35, 0.5, -0.5, 3.0, -3.0], dtype=np.float64)
    rows_g, rows_u = [], []
    for r in range(8):
        gate = g.standard_normal(2 * I // 2) * 2.0
        up = g.standard_normal(2 * I // 2)
        pos = g.permutation(I)[:len(special)]
        gate[pos] = special
        if r == 1:
            up[pos[:6]] = [0.0, -0.0, 1e-30, -1e-30, 1e-38, -1e-38]
        if r == 2:      # the whole row tiny: scale floored, every code a signed zero
            gate *= 1e-31
        if r == 3:      # gate all -0 / +0
            gate = np.where(np.arange(I) % 2 == 0, -0.0, 0.0)
        if r == 4:      # huge gates, tiny ups: finite products
            gate = np.sign(gate) * 1e30
            up = up * 1e-9
        if r == 5:      # negative gates beyond the exp clamp
            gate = -np.abs(gate) * 60.0
        rows_g.append(gate)
        rows_u.append(up)
    gate = np.array(rows_g, dtype=np.float32)
    up = np.array(rows_u, dtype=np.float32)
    gb = W.to_bf16_bits(gate)
    ub = W.to_bf16_bits(up)
    gb[0, :4] = [0x0001, 0x8001, 0x007F, 0x807F]       # bf16 subnormals
    gb[0, 4:6] = [0x8000, 0x0000]
    return np.concatenate([gb, ub], axis=1)


@pytest.mark.parametrize("act_quant", [W.ACT_PER_TENSOR, W.ACT_PER_TOKEN, W.ACT_PER_GROUP])
def test_act_requant_extreme_values(act_quant):
    """SiLU division, bf16 rounding and FP8 encoding at extreme magnitudes: codes
    and scales bit-exact against the oracle."""
    gu = _act_edge_rows()
    M = gu.shape[0]
    seg = np.array([0, 3, M], dtype=np.int32)
    I = gu.shape[1] // 2
    print(f"act_requant extreme values M={M} I={I} mode={act_quant}", flush=True)
    a_ref, s_ref = oracle.act_requant(gu, seg, act_quant)
    a_q, a_s = G.run_act(gu, seg, act_quant)
    assert np.array_equal(a_q[:M], a_ref[:M])
    Gq = 1 if act_quant == W.ACT_PER_TOKEN else -(-I // 128)
    n = 1 if act_quant == W.ACT_PER_TENSOR else M * Gq
    assert np.array_equal(a_s[:n].view(np.uint32), s_ref[:n].view(np.uint32))


@pytest.mark.parametrize("act_quant", [W.ACT_PER_TENSOR, W.ACT_PER_TOKEN, W.ACT_PER_GROUP])
@pytest.mark.parametrize("I", [64, 2048])
def test_act_requant_no_rows(act_quant, I):
    """M = 0 (every segment empty) with m_cap rows present: the per-tensor scale
    is that of an empty maximum (the floored one), bit-exact against the oracle;
    nothing is written past the outputs."""
    g = np.random.default_rng(I)
    m_cap = 21
    seg = np.zeros(4, np.int32)
    gu = W.to_bf16_bits((g.standard_normal((m_cap, 2 * I)) * 1.7).astype(np.float32))
    print(f"act_requant no rows I={I} mode={act_quant}", flush=True)
    a_ref, s_ref = oracle.act_requant(gu, seg, act_quant)
    a_q, a_s = G.run_act(gu, seg, act_quant)
    if act_quant == W.ACT_PER_TENSOR:
        assert a_s[0].view(np.uint32) == s_ref[0].view(np.uint32)


def test_post_reorder_no_local_slot():
    """No slot of any token is local (src2dst all -1): every output row is zero."""
    g = np.random.default_rng(8)
    T, topk, H, m_cap = 9, 8, 7168, 16
    s2d = np.full(T * topk, -1, np.int32)
    w = g.uniform(0.0, 1.0, (T, topk)).astype(np.float32)
    down = W.to_bf16_bits(g.standard_normal((m_cap, H), dtype=np.float32))
    print(f"post_reorder no local slot T={T} topk={topk} H={H}", flush=True)
    ref = oracle.post_reorder(down, s2d, w, T, topk)
    out = G.run_post(down, s2d, w, T, topk)
    assert np.all(ref == 0)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("name", ["dsv3_prefill_ep", "mixtral", "skewed_block"])
def test_act_requant_full_size(name):
    cfg, inp, ids, _ = routed(name)
    s2d, d2s, seg = oracle.permute(ids, cfg.expert_start, cfg.num_local, cfg.m_cap)
    g = np.random.default_rng(2)
    gu = W.to_bf16_bits((g.standard_normal((cfg.m_cap, 2 * cfg.I), dtype=np.float32) * np.float32(1.7)))
    print(f"act_requant full {name} M={seg[-1]} I={cfg.I}", flush=True)
    a_ref, s_ref = oracle.act_requant(gu, seg, cfg.act_quant)
    a_q, a_s = G.run_act(gu, seg, cfg.act_quant)
    M = int(seg[-1])
    assert np.array_equal(a_q[:M], a_ref[:M])
    Gq = 1 if cfg.act_quant == W.ACT_PER_TOKEN else -(-cfg.I // 128)
    n = 1 if cfg.act_quant == W.ACT_PER_TENSOR else M * Gq
    assert np.array_equal(a_s[:n].view(np.uint32), s_ref[:n].view(np.uint32))


# ---- stage 5 ------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "dsv3_prefill_ep", "mixtral", "skewed_block"])
def test_post_reorder(name):
    cfg, inp, ids, w = routed(name)
    s2d, d2s, seg = oracle.permute(ids, cfg.expert_start, cfg.num_local, cfg.m_cap)
    g = np.random.default_rng(4)
    down = W.to_bf16_bits(g.standard_normal((cfg.m_cap, cfg.H), dtype=np.float32))
    print(f"post_reorder {name} T={cfg.T} H={cfg.H}", flush=True)
    ref = oracle.post_reorder(down, s2d, w, cfg.T, cfg.topk)
    out = G.run_post(down, s2d, w, cfg.T, cfg.topk)
    d = np.abs(G.bf16_to_f64(down))
    sd = s2d.reshape(cfg.T, cfg.topk)
    abs_terms = np.zeros((cfg.T, cfg.H))
    for j in range(cfg.topk):
        ok = sd[:, j] >= 0
        abs_terms[ok] += np.abs(w[ok, j].astype(np.float64))[:, None] * d[sd[ok, j]]
    G.assert_sum_close(out, ref, abs_terms, cfg.topk, what="combine", mfma=False)
    none = np.all(s2d.reshape(cfg.T, cfg.topk) < 0, axis=1)
    assert np.all(out[none] == 0)


@pytest.mark.parametrize("topk", [12, 20])
def test_post_reorder_many_slots(topk):
    """topk above 8: up to 16 slots take the 16-slot compacting kernel, more the
    general one; random local slots, some slots non-local (-1), H not a multiple
    of the 1024-column step."""
    g = np.random.default_rng(6)
    T, H = 37, 144
    m_cap = T * topk
    perm = g.permutation(m_cap).astype(np.int32)
    s2d = np.where(g.random(T * topk) < 0.3, -1, perm).astype(np.int32)
    w = g.uniform(0.0, 1.0, (T, topk)).astype(np.float32)
    down = W.to_bf16_bits(g.standard_normal((m_cap, H), dtype=np.float32))
    print(f"post_reorder many slots T={T} topk={topk} H={H}", flush=True)
    ref = oracle.post_reorder(down, s2d, w, T, topk)
    out = G.run_post(down, s2d, w, T, topk)
    d = np.abs(G.bf16_to_f64(down))
    sd = s2d.reshape(T, topk)
    abs_terms = np.zeros((T, H))
    for j in range(topk):
        ok = sd[:, j] >= 0
        abs_terms[ok] += np.abs(w[ok, j].astype(np.float64))[:, None] * d[sd[ok, j]]
    G.assert_sum_close(out, ref, abs_terms, topk, what="combine", mfma=False)
    assert np.all(out[np.all(sd < 0, axis=1)] == 0)
