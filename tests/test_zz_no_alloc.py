"""The allocation-free stage 2 (moe_pre_reorder_quant_noalloc) against the
workspace entry point (moe_pre_reorder_quant), through the C ABI: permutation,
codes and scales bit for bit, on calls in a row that reuse the library's static
scratch, each later one with a smaller input than the first."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_select_amd as moe
import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _routing(g, T, E, topk):
    """Distinct random expert ids per token (global ids 0..E-1)."""
    return np.argsort(g.random((T, E)), axis=1)[:, :topk].astype(np.int32)


def _run(fn_noalloc, x, ids, expert_start, num_local, act_quant):
    T, H = x.shape
    topk = ids.shape[1]
    m_cap = T * min(topk, num_local)
    n_scale = W.a_scale_numel(act_quant, m_cap, H)
    a_q = G.Guarded((m_cap, H), torch.uint8)
    a_s = G.Guarded((n_scale,), torch.float32)
    s2d = G.Guarded((T * topk,), torch.int32)
    d2s = G.Guarded((m_cap,), torch.int32)
    seg = G.Guarded((num_local + 1,), torch.int32)
    xd, idd = G.up_bf16(x), G.up(ids)
    if fn_noalloc:
        moe.moe_pre_reorder_quant_noalloc(xd, idd, a_q.t, a_s.t, s2d.t, d2s.t, seg.t,
                                          expert_start=expert_start, num_local=num_local,
                                          act_quant=act_quant)
    else:
        ws = torch.empty(moe.moe_workspace_bytes(T, topk, num_local), dtype=torch.uint8,
                         device=G.dev())
        moe.moe_pre_reorder_quant(xd, idd, a_q.t, a_s.t, s2d.t, d2s.t, seg.t, ws,
                                  expert_start=expert_start, num_local=num_local,
                                  act_quant=act_quant)
    torch.cuda.synchronize()
    for b, n in ((a_q, "a_q"), (a_s, "a_scale"), (s2d, "src2dst"), (d2s, "dst2src"), (seg, "seg")):
        b.check(n)
    M = int(seg.t[-1].item())
    G_ = 1 if act_quant != W.ACT_PER_GROUP else -(-H // 128)
    n_used = 1 if act_quant == W.ACT_PER_TENSOR else M * G_
    return dict(seg=seg.t.cpu().numpy(), s2d=s2d.t.cpu().numpy(), d2s=d2s.t.cpu().numpy(),
                a_q=a_q.t.cpu().numpy()[:M], a_s=a_s.t.cpu().numpy()[:n_used].view(np.uint32), M=M)


# (T, H, E, topk, expert_start, num_local, act_quant): the first call is the
# DeepSeek-V3 prefill share's shape; each later call is smaller than the first.
# The calls take each way of forming the permutation: separate count and scan
# passes, one count-and-scan block (2048-4096 pairs), one launch (fewer).
CALLS = [(8192, 7168, 256, 8, 0, 32, W.ACT_PER_TOKEN),
         (600, 384, 64, 6, 4, 48, W.ACT_PER_TOKEN),
         (300, 512, 64, 6, 8, 40, W.ACT_PER_GROUP),
         (77, 256, 16, 4, 0, 16, W.ACT_PER_TENSOR)]


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    g = np.random.default_rng(77)
    for i, (T, H, E, topk, start, nl, act) in enumerate(CALLS):
        print(f"noalloc call {i}: T={T} H={H} E={E} topk={topk} local=[{start},{start + nl}) "
              f"act={act}", flush=True)
        x = W.to_bf16_bits(g.standard_normal((T, H), dtype=np.float32))
        ids = _routing(g, T, E, topk)
        got = _run(True, x, ids, start, nl, act)
        ref = _run(False, x, ids, start, nl, act)
        assert got["M"] == ref["M"] and got["M"] > 0
        for k in ("seg", "s2d", "d2s", "a_q", "a_s"):
            assert np.array_equal(got[k], ref[k]), (i, k)
