"""A layer pass captured in a HIP graph and replayed: every replay, with eager
passes and host synchronisations between them, must give the eager result bit
for bit (the kernels are deterministic and the library enqueues nothing but
kernels). Inputs are changed in place between replays to check that a replay
reads the current contents, not a snapshot."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_select_amd as moe
import workloads as W
from tests import gpu_util as G
from tests.test_gpu_layer import small_cfg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["ep_sigmoid_token_channel", "small_fp4_ep", "dsv3_prefill_ep"])
def test_layer_graph_replays_match_eager(name):
    """The full-size prefill share is the configuration the benchmark times from a graph."""
    cfg = W.CONFIGS[name] if name in W.CONFIGS else small_cfg(name)
    print(f"layer graph {name}", flush=True)
    inp = W.gen_layer_inputs(cfg, seed=4)
    x = G.up_bf16(inp.x)
    logits = G.up(inp.logits)
    bias = G.up(inp.bias) if inp.bias is not None else None
    w13, s13 = G.up(inp.w13), G.up(inp.w13_scale.reshape(-1))
    w2, s2 = G.up(inp.w2), G.up(inp.w2_scale.reshape(-1))
    e13 = G.up(inp.w13_e8m0) if inp.w13_e8m0 is not None else None
    e2 = G.up(inp.w2_e8m0) if inp.w2_e8m0 is not None else None
    buf = moe.LayerBuffers.allocate(cfg.T, cfg.H, cfg.I, cfg.topk, cfg.num_local, cfg.act_quant)

    def run():
        moe.layer_forward(x, logits, bias, w13, s13, w2, s2, buf, topk=cfg.topk, n_group=cfg.n_group,
                          topk_group=cfg.topk_group, score_fn=cfg.score_fn, renormalize=cfg.renormalize,
                          routed_scaling_factor=cfg.rsf, apply_rsf=cfg.apply_rsf,
                          expert_start=cfg.expert_start, num_local=cfg.num_local, act_quant=cfg.act_quant,
                          w_quant=cfg.w_quant, w13_e8m0=e13, w2_e8m0=e2)

    graph = moe.LayerGraph(run)
    g = np.random.default_rng(0)
    for rep in range(4 if cfg.T <= 1024 else 3):
        if rep:  # new inputs in place: the replay must see them
            x.copy_(G.up_bf16(W.to_bf16_bits(g.standard_normal(inp.x.shape).astype(np.float32))))
            logits.copy_(G.up(g.standard_normal(inp.logits.shape).astype(np.float32)))
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        eager = [G.bf16_bits(buf.out).copy(), buf.topk_ids.cpu().numpy().copy(), buf.seg_indptr.cpu().numpy().copy()]
        buf.out.zero_()
        buf.topk_ids.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replay = [G.bf16_bits(buf.out), buf.topk_ids.cpu().numpy(), buf.seg_indptr.cpu().numpy()]
        for a, b, what in zip(eager, replay, ["out", "topk_ids", "seg_indptr"]):
            assert np.array_equal(a, b), (rep, what)
