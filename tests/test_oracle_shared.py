"""Pins of the shared-expert extension in the oracle: the appended slots, the
local mapping of shared ids, the permuted layer against the dense per-token
loop, and the fused layer against the sum of a routed-only layer and a
shared-only layer computed separately (a different decomposition of the same
arithmetic, with its own rounding)."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W


def shared_cfg(act_quant=W.ACT_PER_TOKEN, w_quant=W.W_PER_CHANNEL, apply_rsf=1):
    return W.MoEConfig(name="small_shared", T=40, H=256, I=128, E=16, topk=4, num_local=6,
                       expert_start=5, score_fn=W.SCORE_SIGMOID, n_group=4, topk_group=2, rsf=2.5,
                       apply_rsf=apply_rsf, use_bias=True, act_quant=act_quant, w_quant=w_quant,
                       n_shared=1, shared_weight=1.0)


def test_select_appends_shared_slots():
    cfg = shared_cfg()
    inp = W.gen_layer_inputs(cfg, seed=1, weights=False)
    ids, w = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                   cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf, 2, 0.5)
    r_ids, r_w = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                       cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    assert ids.shape == (cfg.T, cfg.topk + 2)
    assert np.array_equal(ids[:, :cfg.topk], r_ids) and np.array_equal(w[:, :cfg.topk], r_w)
    assert np.all(ids[:, cfg.topk:] == np.array([cfg.E, cfg.E + 1])) and np.all(w[:, cfg.topk:] == 0.5)


def test_permute_maps_shared_ids_after_the_routed_experts():
    cfg = shared_cfg()
    inp = W.gen_layer_inputs(cfg, seed=2, weights=False)
    ids, _ = oracle.select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                   cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf, 1, 1.0)
    s2d, d2s, seg = oracle.permute(ids, cfg.expert_start, cfg.num_local, cfg.m_cap, cfg.E, 1)
    assert len(seg) == cfg.num_local + 2
    # the shared expert (local index num_local) holds every token, in token order
    sh = np.arange(seg[cfg.num_local], seg[cfg.num_local + 1])
    assert len(sh) == cfg.T
    assert np.array_equal(d2s[sh], np.arange(cfg.T) * cfg.slots + cfg.topk)
    # routed part identical to the plain permutation of the routed slots (rows shift by nothing:
    # shared rows come after all routed rows)
    s2d_r, d2s_r, seg_r = oracle.permute(np.ascontiguousarray(ids[:, :cfg.topk]), cfg.expert_start,
                                         cfg.num_local, cfg.T * cfg.topk)
    assert np.array_equal(seg[:cfg.num_local + 1], seg_r)
    routed = s2d.reshape(cfg.T, cfg.slots)[:, :cfg.topk].reshape(-1)
    assert np.array_equal(routed, s2d_r)
    # inverse identities
    ok = s2d >= 0
    assert np.array_equal(d2s[s2d[ok]], np.nonzero(ok)[0])


@pytest.mark.parametrize("modes", [(W.ACT_PER_TOKEN, W.W_PER_CHANNEL), (W.ACT_PER_GROUP, W.W_BLOCK)])
def test_dense_equals_permuted_with_shared(modes):
    cfg = shared_cfg(*modes)
    inp = W.gen_layer_inputs(cfg, seed=3)
    res = oracle.layer(inp)
    dense = oracle.dense_layer(inp.x, res["ids"], res["weights"], cfg.I, cfg.expert_start,
                               cfg.num_local, cfg.act_quant, inp.w13, inp.w13_scale, inp.w2,
                               inp.w2_scale, cfg.w_quant, cfg.E, cfg.n_shared)
    assert np.array_equal(dense, res["out"])


def test_fused_equals_routed_plus_shared():
    cfg = shared_cfg()
    inp = W.gen_layer_inputs(cfg, seed=4)
    fused = W.bf16_bits_to_f32(oracle.layer(inp)["out"]).astype(np.float64)
    # routed only: the same layer without the shared slot (its weights dropped)
    rcfg = dataclasses.replace(cfg, n_shared=0)
    rinp = dataclasses.replace(inp, cfg=rcfg, w13=inp.w13[:cfg.num_local], w2=inp.w2[:cfg.num_local],
                               w13_scale=inp.w13_scale[:cfg.num_local],
                               w2_scale=inp.w2_scale[:cfg.num_local])
    routed = W.bf16_bits_to_f32(oracle.layer(rinp)["out"]).astype(np.float64)
    # shared only: every token to one expert (the shared weights) with weight 1
    ids = np.full((cfg.T, 1), cfg.E, np.int32)
    w = np.ones((cfg.T, 1), np.float32)
    shared = W.bf16_bits_to_f32(oracle.dense_layer(
        inp.x, ids, w, cfg.I, cfg.E, 1, cfg.act_quant, inp.w13[cfg.num_local:],
        inp.w13_scale[cfg.num_local:], inp.w2[cfg.num_local:], inp.w2_scale[cfg.num_local:],
        cfg.w_quant)).astype(np.float64)
    ulp = lambda v: np.maximum(np.abs(v), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(fused - (routed + shared)) <= ulp(fused) + ulp(routed) + ulp(shared))
    assert np.abs(shared).max() > 0
