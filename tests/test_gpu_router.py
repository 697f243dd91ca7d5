"""GPU parity of moe_router_select (the router projection before stage 1).

The logits are fp32 sums of bf16 products whose order the matrix cores choose,
so they are compared with the oracle's correctly rounded sums within one fp32
step plus the summation bound. Stage 1 then decides integers from them, so its
parity is checked where both sides take the decision on the same input: the
GPU's ids and weights must equal the oracle's stage 1 applied to the GPU's own
logits (ids bit exact). Against the oracle's stage 1 on the oracle's logits,
tokens may differ only where their selection hinges on a key gap below the
logit error bound; the test counts them and checks each one."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_select_amd as moe
import oracle
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def run_router(x_bits, wg_bits, bias, cfg):
    T, H = x_bits.shape
    E = wg_bits.shape[0]
    logits = G.Guarded((T, E), torch.float32)
    ids = G.Guarded((T, cfg.topk), torch.int32)
    w = G.Guarded((T, cfg.topk), torch.float32)
    moe.moe_router_select(G.up_bf16(x_bits), G.up_bf16(wg_bits), G.up(bias) if bias is not None else None,
                          logits.t, ids.t, w.t, topk=cfg.topk, n_group=cfg.n_group,
                          topk_group=cfg.topk_group, score_fn=cfg.score_fn, renormalize=cfg.renormalize,
                          routed_scaling_factor=cfg.rsf, apply_rsf=cfg.apply_rsf)
    torch.cuda.synchronize()
    for g, n in [(logits, "logits"), (ids, "topk_ids"), (w, "topk_weights")]:
        g.check(n)
    return logits.t.cpu().numpy(), ids.t.cpu().numpy(), w.t.cpu().numpy()


def check_logits(got, ref, x_bits, wg_bits):
    xf = np.abs(W.bf16_bits_to_f32(x_bits).astype(np.float64))
    wf = np.abs(W.bf16_bits_to_f32(wg_bits).astype(np.float64))
    abs_terms = xf @ wf.T
    H = x_bits.shape[1]
    # fp32 accumulation of exact products in an unspecified order, 32 per MFMA
    bound = np.spacing(np.abs(ref)).astype(np.float64) + (H * 2.0 ** -24 + (H // 32 + 1) * 2.0 ** -13) * abs_terms
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bound), f"logits: worst excess {(err - bound).max():.3g}"
    return float((err / np.maximum(abs_terms, 1e-30)).max()), bound


@pytest.mark.parametrize("name", ["tiny", "dsv3_decode_ep", "dsv3_prefill_ep", "mixtral"])
def test_router_select_workloads(name):
    cfg = W.CONFIGS[name]
    x = W.gen_tokens(cfg)
    wg = W.gen_router_bf16(cfg)
    bias = W.gen_bias(cfg)
    print(f"router_select {name} T={cfg.T} H={cfg.H} E={cfg.E}", flush=True)
    logits, ids, w = run_router(x, wg, bias, cfg)
    ref_logits = oracle.router_logits(x, wg)
    worst, bound = check_logits(logits, ref_logits, x, wg)
    # stage 1 on the GPU's own logits: exact
    ids_own, w_own = oracle.select_experts(logits, bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                           cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    assert np.array_equal(ids, ids_own)
    assert np.all(np.abs(w.astype(np.float64) - w_own) <= 4e-6 * np.abs(w_own) + 1e-30)
    # against the oracle's own logits: differences only at near-ties
    ids_ref, _ = oracle.select_experts(ref_logits, bias, cfg.topk, cfg.n_group, cfg.topk_group,
                                       cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf)
    diff = np.nonzero(np.any(np.sort(ids, 1) != np.sort(ids_ref, 1), axis=1))[0]
    print(f"{name}: worst logit error / sum|x w| {worst:.3g}; {len(diff)} of {cfg.T} tokens select "
          f"a different set than on the oracle's logits", flush=True)
    assert len(diff) <= max(1, cfg.T // 200)
    for t in diff:
        # every expert in exactly one of the two sets has a logit within twice the
        # error bound of some expert in the other set (a near-tie)
        a, b = set(ids[t]) - set(ids_ref[t]), set(ids_ref[t]) - set(ids[t])
        for e in a | b:
            other = b if e in a else a
            assert min(abs(float(ref_logits[t, e]) - float(ref_logits[t, o])) for o in other) <= \
                2 * max(bound[t, e], max(bound[t, o] for o in other)), (t, e)


def test_router_ragged_shapes():
    """T not a multiple of 64, E not a multiple of 128, H not a multiple of 64."""
    g = np.random.default_rng(4)
    cfg = W.CONFIGS["tiny"]
    import dataclasses
    cfg = dataclasses.replace(cfg, T=77, H=200, E=12, topk=3)
    x = W.to_bf16_bits(g.standard_normal((cfg.T, cfg.H)).astype(np.float32))
    wg = W.to_bf16_bits((g.standard_normal((cfg.E, cfg.H)) * 0.05).astype(np.float32))
    print("router ragged T=77 H=200 E=12", flush=True)
    logits, ids, w = run_router(x, wg, None, cfg)
    check_logits(logits, oracle.router_logits(x, wg), x, wg)
    ids_own, _ = oracle.select_experts(logits, None, cfg.topk, 1, 1, cfg.score_fn, cfg.renormalize,
                                       cfg.rsf, cfg.apply_rsf)
    assert np.array_equal(ids, ids_own)
