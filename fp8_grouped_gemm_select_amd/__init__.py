"""Python binding of libmoe, the MI355X (gfx950) EP-MoE FP8 hot path.

Thin ctypes marshalling over the C ABI declared in ``include/moe.h``: each
function takes torch tensors that already live on the GPU, checks dtypes and
devices, and passes raw pointers, sizes and the current HIP stream. Every step
of the computation runs in the HIP kernels of ``libmoe.so``; nothing here
computes. If the library is not built, loading fails with an error (build it
with ``python -m fp8_grouped_gemm_select_amd._build`` or
``__graft_entry__.build()``).

Error codes become exceptions: NULL / bad argument / shape / workspace ->
ValueError, unsupported combination -> NotImplementedError, HIP launch error ->
RuntimeError. All arguments after the tensors are keyword-only.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_INVALID_ARG, MOE_ERR_SHAPE = 0, -1, -2, -3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = -4, -5, -6
MOE_NOALLOC_SCRATCH_BYTES = 8 << 20  # static scratch of moe_pre_reorder_quant_noalloc (moe.h)

SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
ACT_PER_TENSOR, ACT_PER_TOKEN, ACT_PER_GROUP = 0, 1, 2
W_PER_EXPERT, W_PER_CHANNEL, W_BLOCK = 0, 1, 2

EXPORTS = ["moe_select_experts", "moe_workspace_bytes", "moe_pre_reorder_quant",
           "moe_grouped_gemm_fp8", "moe_act_requant", "moe_post_reorder", "moe_status_string",
           "moe_router_select", "moe_select_experts_shared", "moe_pre_reorder_quant_shared",
           "moe_grouped_gemm_mxfp4", "moe_router_workspace_bytes",
           "moe_pre_reorder_quant_noalloc"]

_lib = None


class MoEError(RuntimeError):
    pass


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmoe.so is not built ({LIB_PATH}); run "
                           "`python -m fp8_grouped_gemm_select_amd._build` first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.moe_select_experts.restype = ctypes.c_int
    lib.moe_select_experts.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I32, F32, I32, P, P, P]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_workspace_bytes.argtypes = [I64, I32, I32]
    lib.moe_pre_reorder_quant.restype = ctypes.c_int
    lib.moe_pre_reorder_quant.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I64, P, P, I64,
                                          P, P, P, P, SZ, P]
    lib.moe_pre_reorder_quant_noalloc.restype = ctypes.c_int
    lib.moe_pre_reorder_quant_noalloc.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I64, P, P,
                                                  I64, P, P, P, P]
    lib.moe_grouped_gemm_fp8.restype = ctypes.c_int
    lib.moe_grouped_gemm_fp8.argtypes = [P, P, I64, I32, P, P, I64, I32, P, I32, I64, I32, I32,
                                         P, P]
    lib.moe_grouped_gemm_mxfp4.restype = ctypes.c_int
    lib.moe_grouped_gemm_mxfp4.argtypes = [P, P, I64, I32, P, P, P, I64, I32, P, I32, I64, I32, I32,
                                           P, P]
    lib.moe_act_requant.restype = ctypes.c_int
    lib.moe_act_requant.argtypes = [P, P, I32, I64, I32, I32, P, P, I64, P, SZ, P]
    lib.moe_post_reorder.restype = ctypes.c_int
    lib.moe_post_reorder.argtypes = [P, P, P, I64, I32, I32, I64, P, P]
    lib.moe_select_experts_shared.restype = ctypes.c_int
    lib.moe_select_experts_shared.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I32, F32, I32, I32,
                                              F32, P, P, P]
    lib.moe_pre_reorder_quant_shared.restype = ctypes.c_int
    lib.moe_pre_reorder_quant_shared.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I32, I32, I64, P,
                                                 P, I64, P, P, P, P, SZ, P]
    lib.moe_router_select.restype = ctypes.c_int
    lib.moe_router_select.argtypes = [P, P, P, I64, I32, I32, I32, I32, I32, I32, I32, F32, I32, P, P,
                                      P, P, SZ, P]
    lib.moe_router_workspace_bytes.restype = SZ
    lib.moe_router_workspace_bytes.argtypes = [I64, I32, I32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _check(rc: int, fn: str) -> None:
    if rc == MOE_OK:
        return
    msg = f"{fn}: {load_library().moe_status_string(rc).decode()}"
    if rc == MOE_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if rc == MOE_ERR_HIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else ctypes.c_void_p(t.data_ptr() or 0)


def _dtype(t, *dts, name="tensor"):
    if t is not None and t.dtype not in dts:
        raise TypeError(f"{name} must be one of {dts}, got {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def status_string(code: int) -> str:
    return load_library().moe_status_string(int(code)).decode()


def moe_workspace_bytes(T: int, topk: int, num_local: int) -> int:
    return int(load_library().moe_workspace_bytes(int(T), int(topk), int(num_local)))


def moe_select_experts(logits, correction_bias, topk_ids, topk_weights, *, topk, n_group=1,
                       topk_group=1, score_fn=SCORE_SOFTMAX, renormalize=1,
                       routed_scaling_factor=1.0, apply_rsf=1, stream=None):
    _dtype(logits, torch.float32, name="logits")
    _dtype(correction_bias, torch.float32, name="correction_bias")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(topk_weights, torch.float32, name="topk_weights")
    T, E = logits.shape
    rc = load_library().moe_select_experts(
        _ptr(logits), _ptr(correction_bias), T, E, topk, n_group, topk_group, score_fn,
        renormalize, float(routed_scaling_factor), apply_rsf, _ptr(topk_ids), _ptr(topk_weights),
        _stream(stream))
    _check(rc, "moe_select_experts")


def moe_router_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(load_library().moe_router_workspace_bytes(T, H, E))


def moe_router_select(x, wg, correction_bias, logits, topk_ids, topk_weights, *, topk, n_group=1,
                      topk_group=1, score_fn=SCORE_SOFTMAX, renormalize=1,
                      routed_scaling_factor=1.0, apply_rsf=1, workspace=None, stream=None):
    """Router projection logits = x @ wg^T (x bf16 [T, H], wg bf16 [E, H]) into
    `logits` (fp32 [T, E]), then stage 1 on them. `workspace`: a device byte
    tensor of at least moe_router_workspace_bytes(T, H, E) (allocated here when
    omitted)."""
    _dtype(x, torch.bfloat16, name="x")
    _dtype(wg, torch.bfloat16, name="wg")
    _dtype(correction_bias, torch.float32, name="correction_bias")
    _dtype(logits, torch.float32, name="logits")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(topk_weights, torch.float32, name="topk_weights")
    T, H = x.shape
    E = wg.shape[0]
    if wg.shape[1] != H or tuple(logits.shape) != (T, E):
        raise MoEError("moe_router_select: shapes of x, wg and logits disagree")
    need = moe_router_workspace_bytes(T, H, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load_library().moe_router_select(
        _ptr(x), _ptr(wg), _ptr(correction_bias), T, H, E, topk, n_group, topk_group, score_fn,
        renormalize, float(routed_scaling_factor), apply_rsf, _ptr(logits), _ptr(topk_ids),
        _ptr(topk_weights), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "moe_router_select")


def moe_select_experts_shared(logits, correction_bias, topk_ids, topk_weights, *, topk, n_shared,
                              shared_weight, n_group=1, topk_group=1, score_fn=SCORE_SOFTMAX,
                              renormalize=1, routed_scaling_factor=1.0, apply_rsf=1, stream=None):
    """Stage 1 plus n_shared always-selected slots per token (ids E.., weight
    shared_weight): topk_ids / topk_weights are [T, topk + n_shared]."""
    _dtype(logits, torch.float32, name="logits")
    _dtype(correction_bias, torch.float32, name="correction_bias")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(topk_weights, torch.float32, name="topk_weights")
    T, E = logits.shape
    if topk_ids.shape[1] != topk + n_shared or topk_weights.shape[1] != topk + n_shared:
        raise MoEError("moe_select_experts_shared: outputs need topk + n_shared columns")
    rc = load_library().moe_select_experts_shared(
        _ptr(logits), _ptr(correction_bias), T, E, topk, n_group, topk_group, score_fn,
        renormalize, float(routed_scaling_factor), apply_rsf, n_shared, float(shared_weight),
        _ptr(topk_ids), _ptr(topk_weights), _stream(stream))
    _check(rc, "moe_select_experts_shared")


def moe_pre_reorder_quant_shared(x, topk_ids, a_q, a_scale, src2dst, dst2src, seg_indptr, workspace,
                                 *, expert_start, num_routed, shared_base, n_shared, act_quant,
                                 stream=None):
    """Stage 2 with shared experts: ids in [shared_base, shared_base + n_shared) are
    local experts num_routed.. (seg_indptr has num_routed + n_shared + 1 entries)."""
    _dtype(x, torch.bfloat16, name="x")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(a_q, torch.uint8, torch.float8_e4m3fn, name="a_q")
    _dtype(a_scale, torch.float32, name="a_scale")
    T, H = x.shape
    topk = topk_ids.shape[1]
    m_cap = a_q.shape[0]
    rc = load_library().moe_pre_reorder_quant_shared(
        _ptr(x), _ptr(topk_ids), T, H, topk, expert_start, num_routed, shared_base, n_shared,
        act_quant, m_cap, _ptr(a_q), _ptr(a_scale), a_scale.numel(), _ptr(src2dst), _ptr(dst2src),
        _ptr(seg_indptr), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(rc, "moe_pre_reorder_quant_shared")


def moe_pre_reorder_quant(x, topk_ids, a_q, a_scale, src2dst, dst2src, seg_indptr, workspace, *,
                          expert_start, num_local, act_quant, stream=None):
    _dtype(x, torch.bfloat16, name="x")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(a_q, torch.uint8, torch.float8_e4m3fn, name="a_q")
    _dtype(a_scale, torch.float32, name="a_scale")
    T, H = x.shape
    topk = topk_ids.shape[1]
    m_cap = a_q.shape[0]
    rc = load_library().moe_pre_reorder_quant(
        _ptr(x), _ptr(topk_ids), T, H, topk, expert_start, num_local, act_quant, m_cap,
        _ptr(a_q), _ptr(a_scale), a_scale.numel(), _ptr(src2dst), _ptr(dst2src),
        _ptr(seg_indptr), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(rc, "moe_pre_reorder_quant")


def moe_pre_reorder_quant_noalloc(x, topk_ids, a_q, a_scale, src2dst, dst2src, seg_indptr, *,
                                  expert_start, num_local, act_quant, stream=None):
    """moe_pre_reorder_quant with the library's static scratch instead of a
    workspace: nothing is allocated. Calls that overlap on one GPU race."""
    _dtype(x, torch.bfloat16, name="x")
    _dtype(topk_ids, torch.int32, name="topk_ids")
    _dtype(a_q, torch.uint8, torch.float8_e4m3fn, name="a_q")
    _dtype(a_scale, torch.float32, name="a_scale")
    T, H = x.shape
    topk = topk_ids.shape[1]
    m_cap = a_q.shape[0]
    rc = load_library().moe_pre_reorder_quant_noalloc(
        _ptr(x), _ptr(topk_ids), T, H, topk, expert_start, num_local, act_quant, m_cap,
        _ptr(a_q), _ptr(a_scale), a_scale.numel(), _ptr(src2dst), _ptr(dst2src),
        _ptr(seg_indptr), _stream(stream))
    _check(rc, "moe_pre_reorder_quant_noalloc")


def moe_grouped_gemm_fp8(a_q, a_scale, b_q, b_scale, seg_indptr, c, *, act_quant, w_quant,
                         stream=None):
    _dtype(a_q, torch.uint8, torch.float8_e4m3fn, name="a_q")
    _dtype(b_q, torch.uint8, torch.float8_e4m3fn, name="b_q")
    _dtype(c, torch.bfloat16, name="c")
    m_cap, K = a_q.shape
    num_local, N, K2 = b_q.shape
    if K2 != K:
        raise ValueError("a_q and b_q disagree on K")
    rc = load_library().moe_grouped_gemm_fp8(
        _ptr(a_q), _ptr(a_scale), a_scale.numel(), act_quant, _ptr(b_q), _ptr(b_scale),
        b_scale.numel(), w_quant, _ptr(seg_indptr), num_local, m_cap, N, K, _ptr(c),
        _stream(stream))
    _check(rc, "moe_grouped_gemm_fp8")


def moe_grouped_gemm_mxfp4(a_q, a_scale, b_fp4, b_e8m0, b_scale, seg_indptr, c, *, act_quant, w_quant,
                           stream=None):
    """Stage 3 with MXFP4 weights: b_fp4 uint8 [E_l, N, K/2] packed E2M1 codes,
    b_e8m0 uint8 [E_l, N, K/32] block scales, b_scale fp32 factor."""
    _dtype(a_q, torch.uint8, torch.float8_e4m3fn, name="a_q")
    _dtype(b_fp4, torch.uint8, name="b_fp4")
    _dtype(b_e8m0, torch.uint8, name="b_e8m0")
    _dtype(c, torch.bfloat16, name="c")
    m_cap, K = a_q.shape
    num_local, N, Kh = b_fp4.shape
    if 2 * Kh != K or tuple(b_e8m0.shape) != (num_local, N, K // 32):
        raise ValueError("a_q, b_fp4 and b_e8m0 disagree on K")
    rc = load_library().moe_grouped_gemm_mxfp4(
        _ptr(a_q), _ptr(a_scale), a_scale.numel(), act_quant, _ptr(b_fp4), _ptr(b_e8m0), _ptr(b_scale),
        b_scale.numel(), w_quant, _ptr(seg_indptr), num_local, m_cap, N, K, _ptr(c), _stream(stream))
    _check(rc, "moe_grouped_gemm_mxfp4")


def moe_act_requant(gateup, seg_indptr, a_q, a_scale, workspace, *, act_quant, stream=None):
    _dtype(gateup, torch.bfloat16, name="gateup")
    m_cap, two_i = gateup.shape
    rc = load_library().moe_act_requant(
        _ptr(gateup), _ptr(seg_indptr), seg_indptr.numel() - 1, m_cap, two_i // 2, act_quant,
        _ptr(a_q), _ptr(a_scale), a_scale.numel(), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_act_requant")


def moe_post_reorder(down, src2dst, topk_weights, out, *, stream=None):
    _dtype(down, torch.bfloat16, name="down")
    _dtype(out, torch.bfloat16, name="out")
    T, H = out.shape
    topk = topk_weights.shape[1]
    rc = load_library().moe_post_reorder(
        _ptr(down), _ptr(src2dst), _ptr(topk_weights), T, H, topk, down.shape[0], _ptr(out),
        _stream(stream))
    _check(rc, "moe_post_reorder")


from .layer import LayerBuffers, LayerGraph, layer_forward  # noqa: E402
