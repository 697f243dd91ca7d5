"""End-to-end GPU parity: the whole layer (five stages through the C ABI) against
the CPU oracle on the same seeded inputs.

Ids and permutation bit-exact; the bf16 layer output within atol 1e-2 + rtol
2e-2. Small ragged layers are compared in full; the full-size workloads on
sampled tokens recomputed by the oracle's dense per-token loop. Also: two runs
are bitwise identical, and experts with no tokens are never read.
"""
import dataclasses

import numpy as np
import pytest
import torch

import fp8_grouped_gemm_select_amd as moe
import oracle
import workloads as W
from tests import gpu_util as G
from tests.test_oracle_layer import small_cfg, LAYER_CASES

pytestmark = pytest.mark.gpu


def run_layer(inp, w13_dev=None, w2_dev=None):
    cfg = inp.cfg
    buf = moe.LayerBuffers.allocate(cfg.T, cfg.H, cfg.I, cfg.topk, cfg.num_local, cfg.act_quant)
    w13 = w13_dev if w13_dev is not None else G.up(inp.w13)
    w2 = w2_dev if w2_dev is not None else G.up(inp.w2)
    moe.layer_forward(G.up_bf16(inp.x), G.up(inp.logits),
                      G.up(inp.bias) if inp.bias is not None else None,
                      w13, G.up(inp.w13_scale.reshape(-1)), w2, G.up(inp.w2_scale.reshape(-1)), buf,
                      topk=cfg.topk, n_group=cfg.n_group, topk_group=cfg.topk_group,
                      score_fn=cfg.score_fn, renormalize=cfg.renormalize,
                      routed_scaling_factor=cfg.rsf, apply_rsf=cfg.apply_rsf,
                      expert_start=cfg.expert_start, num_local=cfg.num_local,
                      act_quant=cfg.act_quant, w_quant=cfg.w_quant)
    torch.cuda.synchronize()
    return buf


@pytest.mark.parametrize("name", ["tiny"] + LAYER_CASES)
def test_layer_small_full_compare(name):
    cfg = W.CONFIGS["tiny"] if name == "tiny" else small_cfg(name)
    inp = W.gen_layer_inputs(cfg, seed=3)
    print(f"layer {name} T={cfg.T} H={cfg.H} I={cfg.I}", flush=True)
    ref = oracle.layer(inp)
    buf = run_layer(inp)
    assert np.array_equal(buf.topk_ids.cpu().numpy(), ref["ids"])
    assert np.array_equal(buf.seg_indptr.cpu().numpy(), ref["seg_indptr"])
    assert np.array_equal(buf.src2dst.cpu().numpy(), ref["src2dst"])
    assert np.array_equal(buf.dst2src.cpu().numpy(), ref["dst2src"])
    M = int(ref["seg_indptr"][-1])
    assert np.array_equal(buf.a13.cpu().numpy()[:M], ref["a13"][:M])
    G.assert_close_layer(G.bf16_bits(buf.out), ref["out"], what="layer output")


@pytest.mark.parametrize("name", ["tiny", "skew_group_block"])
def test_layer_deterministic(name):
    cfg = W.CONFIGS["tiny"] if name == "tiny" else small_cfg(name)
    inp = W.gen_layer_inputs(cfg, seed=9)
    print(f"layer determinism {name}", flush=True)
    a = run_layer(inp)
    o1 = G.bf16_bits(a.out).copy()
    c1 = G.bf16_bits(a.c13).copy()
    b = run_layer(inp)
    assert np.array_equal(o1, G.bf16_bits(b.out))
    M = int(a.seg_indptr[-1].item())
    assert np.array_equal(c1[:M], G.bf16_bits(b.c13)[:M])


def test_layer_empty_experts_never_read():
    cfg = small_cfg("skew_group_block")
    inp = W.gen_layer_inputs(cfg, seed=5)
    ref = oracle.layer(inp)
    seg = ref["seg_indptr"]
    empty = [e for e in range(cfg.num_local) if seg[e] == seg[e + 1]]
    assert empty
    print(f"layer empty experts {empty}", flush=True)
    a = G.bf16_bits(run_layer(inp).out).copy()
    w13, w2 = inp.w13.copy(), inp.w2.copy()
    w13[empty] = 0x7F
    w2[empty] = 0x7F
    s13, s2 = inp.w13_scale.copy(), inp.w2_scale.copy()
    s13[empty] = np.nan
    s2[empty] = np.nan
    b = G.bf16_bits(run_layer(dataclasses.replace(inp, w13=w13, w2=w2, w13_scale=s13,
                                                   w2_scale=s2)).out)
    assert np.array_equal(a, b)


def test_layer_rsf_scales_output_once():
    cfg = small_cfg("ep_sigmoid_token_channel")
    inp = W.gen_layer_inputs(cfg, seed=7)
    print("layer rsf 2.5 vs 1.0", flush=True)
    o25 = G.bf16_to_f64(G.bf16_bits(run_layer(inp).out))
    inp1 = dataclasses.replace(inp, cfg=dataclasses.replace(cfg, rsf=1.0))
    o1 = G.bf16_to_f64(G.bf16_bits(run_layer(inp1).out))
    assert np.all(np.abs(o25 - 2.5 * o1) <= np.abs(o25) * 2.0 ** -7 + 1e-30)


@pytest.mark.parametrize("name", ["dsv3_decode_ep", "dsv3_prefill_ep", "skewed_block"])
def test_layer_full_size_sampled_tokens(name):
    """Full workload in the benchmark's launch configuration: routing and
    permutation compared in full, the output on 24 sampled tokens recomputed by
    the dense per-token oracle."""
    cfg = W.CONFIGS[name]
    inp = W.gen_layer_inputs(cfg, seed=0)
    print(f"layer full {name} T={cfg.T}", flush=True)
    buf = run_layer(inp)
    ids_ref, w_ref = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group,
                                           cfg.topk_group, cfg.score_fn, cfg.renormalize,
                                           cfg.rsf, cfg.apply_rsf)
    ids = buf.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    s2d, d2s, seg = oracle.permute(ids_ref, cfg.expert_start, cfg.num_local, cfg.m_cap)
    assert np.array_equal(buf.seg_indptr.cpu().numpy(), seg)
    assert np.array_equal(buf.src2dst.cpu().numpy(), s2d)
    g = np.random.default_rng(5)
    local_tok = np.nonzero(np.any(s2d.reshape(cfg.T, cfg.topk) >= 0, axis=1))[0]
    toks = np.unique(np.concatenate([g.choice(local_tok, 20, replace=False), [0, cfg.T - 1]]))
    w = buf.topk_weights.cpu().numpy()
    ref = oracle.dense_layer(inp.x[toks], ids_ref[toks], w_ref[toks], cfg.I, cfg.expert_start,
                             cfg.num_local, cfg.act_quant, inp.w13, inp.w13_scale, inp.w2,
                             inp.w2_scale, cfg.w_quant)
    out = G.bf16_bits(buf.out)[toks]
    G.assert_close_layer(out, ref, what=f"{name} sampled tokens")
    assert np.all(np.abs(w[toks].astype(np.float64) - w_ref[toks]) <= 4e-6 * np.abs(w_ref[toks]))
