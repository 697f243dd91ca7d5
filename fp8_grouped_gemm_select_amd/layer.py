"""One EP-MoE layer forward on one GPU: the five libmoe stages in order.

Buffers are allocated once (``LayerBuffers``) with torch, sized for the worst
case (m_cap = T * min(topk, num_local) local rows), and reused by every call;
``layer_forward`` only enqueues the five C-ABI calls on the current stream and
never synchronises. The data-dependent row count M stays on the device in
``seg_indptr[num_local]``.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (moe_act_requant, moe_grouped_gemm_fp8, moe_grouped_gemm_mxfp4, moe_post_reorder,
               moe_pre_reorder_quant,
               moe_pre_reorder_quant_shared, moe_select_experts, moe_select_experts_shared,
               moe_workspace_bytes, ACT_PER_GROUP, ACT_PER_TENSOR, ACT_PER_TOKEN)


def _scale_numel(act_quant: int, m_cap: int, K: int) -> int:
    if act_quant == ACT_PER_TENSOR:
        return 1
    if act_quant == ACT_PER_TOKEN:
        return m_cap
    return m_cap * (-(-K // 128))


@dataclasses.dataclass
class LayerBuffers:
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    src2dst: torch.Tensor
    dst2src: torch.Tensor
    seg_indptr: torch.Tensor
    a13: torch.Tensor
    a13_scale: torch.Tensor
    c13: torch.Tensor
    a2: torch.Tensor
    a2_scale: torch.Tensor
    c2: torch.Tensor
    out: torch.Tensor
    workspace: torch.Tensor

    @staticmethod
    def allocate(T, H, I, topk, num_local, act_quant, device="cuda", n_shared=0):
        """Worst-case buffers; with n_shared shared experts every token has
        topk + n_shared slots over num_local + n_shared local experts."""
        topk, num_local = topk + n_shared, num_local + n_shared
        m_cap = T * min(topk, num_local)
        dev = torch.device(device)
        ws = moe_workspace_bytes(T, topk, num_local)
        return LayerBuffers(
            topk_ids=torch.empty((T, topk), dtype=torch.int32, device=dev),
            topk_weights=torch.empty((T, topk), dtype=torch.float32, device=dev),
            src2dst=torch.empty(T * topk, dtype=torch.int32, device=dev),
            dst2src=torch.empty(m_cap, dtype=torch.int32, device=dev),
            seg_indptr=torch.empty(num_local + 1, dtype=torch.int32, device=dev),
            a13=torch.empty((m_cap, H), dtype=torch.uint8, device=dev),
            a13_scale=torch.empty(_scale_numel(act_quant, m_cap, H), dtype=torch.float32, device=dev),
            c13=torch.empty((m_cap, 2 * I), dtype=torch.bfloat16, device=dev),
            a2=torch.empty((m_cap, I), dtype=torch.uint8, device=dev),
            a2_scale=torch.empty(_scale_numel(act_quant, m_cap, I), dtype=torch.float32, device=dev),
            c2=torch.empty((m_cap, H), dtype=torch.bfloat16, device=dev),
            out=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
            workspace=torch.empty(max(ws, 256), dtype=torch.uint8, device=dev),
        )


def layer_forward(x, logits, correction_bias, w13, w13_scale, w2, w2_scale, buf: LayerBuffers, *,
                  topk, n_group, topk_group, score_fn, renormalize, routed_scaling_factor,
                  apply_rsf, expert_start, num_local, act_quant, w_quant, n_shared=0,
                  shared_weight=1.0, w13_e8m0=None, w2_e8m0=None, stream=None):
    """x bf16 [T,H], logits fp32 [T,E]; w13 e4m3 [E_l,2I,H]; w2 e4m3 [E_l,H,I]. Result in buf.out.

    With n_shared > 0 the shared experts are the last n_shared entries of w13 /
    w2 (E_l = num_local + n_shared) and every token also takes them with
    weight shared_weight, inside the same grouped GEMMs.
    With w13_e8m0 / w2_e8m0 given, w13 / w2 are MXFP4 (packed E2M1 [E_l,N,K/2])
    with those E8M0 block scales, and w13_scale / w2_scale the fp32 factors."""
    if n_shared:
        moe_select_experts_shared(logits, correction_bias, buf.topk_ids, buf.topk_weights,
                                  topk=topk, n_shared=n_shared, shared_weight=shared_weight,
                                  n_group=n_group, topk_group=topk_group, score_fn=score_fn,
                                  renormalize=renormalize,
                                  routed_scaling_factor=routed_scaling_factor,
                                  apply_rsf=apply_rsf, stream=stream)
        moe_pre_reorder_quant_shared(x, buf.topk_ids, buf.a13, buf.a13_scale, buf.src2dst,
                                     buf.dst2src, buf.seg_indptr, buf.workspace,
                                     expert_start=expert_start, num_routed=num_local,
                                     shared_base=logits.shape[1], n_shared=n_shared,
                                     act_quant=act_quant, stream=stream)
    else:
        moe_select_experts(logits, correction_bias, buf.topk_ids, buf.topk_weights, topk=topk,
                           n_group=n_group, topk_group=topk_group, score_fn=score_fn,
                           renormalize=renormalize, routed_scaling_factor=routed_scaling_factor,
                           apply_rsf=apply_rsf, stream=stream)
        moe_pre_reorder_quant(x, buf.topk_ids, buf.a13, buf.a13_scale, buf.src2dst, buf.dst2src,
                              buf.seg_indptr, buf.workspace, expert_start=expert_start,
                              num_local=num_local, act_quant=act_quant, stream=stream)
    if w13_e8m0 is not None:
        moe_grouped_gemm_mxfp4(buf.a13, buf.a13_scale, w13, w13_e8m0, w13_scale, buf.seg_indptr, buf.c13,
                               act_quant=act_quant, w_quant=w_quant, stream=stream)
    else:
        moe_grouped_gemm_fp8(buf.a13, buf.a13_scale, w13, w13_scale, buf.seg_indptr, buf.c13,
                             act_quant=act_quant, w_quant=w_quant, stream=stream)
    moe_act_requant(buf.c13, buf.seg_indptr, buf.a2, buf.a2_scale, buf.workspace,
                    act_quant=act_quant, stream=stream)
    if w2_e8m0 is not None:
        moe_grouped_gemm_mxfp4(buf.a2, buf.a2_scale, w2, w2_e8m0, w2_scale, buf.seg_indptr, buf.c2,
                               act_quant=act_quant, w_quant=w_quant, stream=stream)
    else:
        moe_grouped_gemm_fp8(buf.a2, buf.a2_scale, w2, w2_scale, buf.seg_indptr, buf.c2,
                             act_quant=act_quant, w_quant=w_quant, stream=stream)
    moe_post_reorder(buf.c2, buf.src2dst, buf.topk_weights, buf.out, stream=stream)
    return buf.out


class LayerGraph:
    """One layer pass captured in a HIP graph (torch.cuda.CUDAGraph) for replay.

    `fn` enqueues the pass (e.g. a closure over layer_forward with fixed
    tensors); it runs `warmup` times on a side stream of default priority first
    (the library caches device attributes on its first call), then once under
    capture. Every replay reuses the captured device addresses, so the inputs
    are updated in place between replays. The library enqueues no memset, copy
    or allocation, so the graph holds only its kernels."""

    def __init__(self, fn, warmup: int = 2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()

    def replay(self):
        self.graph.replay()
