"""CPU oracle for the EP-MoE FP8 hot path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package. The product library never touches it. It wraps
``liboracle.so`` (plain C loops in ``oracle.c``, built by ``build.py``) with
numpy in / numpy out functions, one per stage of the layer, plus the dense
per-token layer and the number-format primitives.

Each function follows the passage cited in ``oracle.c``. Pins live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

FLAG_SCALE_A_BY_EXPERT = 1  # planted defect: scale_a indexed by expert id (mutation tests)

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [F32]
    lib.oracle_e4m3_decode.restype = F32
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne.argtypes = [F32]
    lib.oracle_bf16_rne_f64.restype = ctypes.c_uint16
    lib.oracle_bf16_rne_f64.argtypes = [ctypes.c_double]
    lib.oracle_exp_ref.restype = F32
    lib.oracle_exp_ref.argtypes = [F32]
    lib.oracle_math_vec.restype = ctypes.c_int
    lib.oracle_math_vec.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.oracle_sigmoid.restype = F32
    lib.oracle_sigmoid.argtypes = [F32]
    lib.oracle_silu_mul_bf16.restype = ctypes.c_uint16
    lib.oracle_silu_mul_bf16.argtypes = [F32, F32]
    lib.oracle_select_experts.restype = ctypes.c_int
    lib.oracle_select_experts.argtypes = [P, P, I64, I32, I32, I32, I32, I32, I32, F32, I32, P, P]
    lib.oracle_permute.restype = ctypes.c_int
    lib.oracle_permute.argtypes = [P, I64, I32, I32, I32, I64, P, P, P]
    lib.oracle_pre_reorder_quant.restype = ctypes.c_int
    lib.oracle_pre_reorder_quant.argtypes = [P, P, I64, I32, I32, I32, P, P]
    lib.oracle_grouped_gemm.restype = ctypes.c_int
    lib.oracle_grouped_gemm.argtypes = [P, P, I32, P, P, I32, P, I32, I32, I32, P, I32]
    lib.oracle_grouped_gemm_rows.restype = ctypes.c_int
    lib.oracle_grouped_gemm_rows.argtypes = [P, P, I32, P, P, I32, P, I32, I32, I32, P, I64, P]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_grouped_gemm_mxfp4.restype = ctypes.c_int
    lib.oracle_grouped_gemm_mxfp4.argtypes = [P, P, I32, P, P, P, I32, P, I32, I32, I32, P]
    lib.oracle_grouped_gemm_mxfp4_rows.restype = ctypes.c_int
    lib.oracle_grouped_gemm_mxfp4_rows.argtypes = [P, P, I32, P, P, P, I32, P, I32, I32, I32, P, I64, P]
    lib.oracle_act_requant.restype = ctypes.c_int
    lib.oracle_act_requant.argtypes = [P, P, I32, I32, I32, P, P]
    lib.oracle_router_logits.restype = ctypes.c_int
    lib.oracle_router_logits.argtypes = [P, P, I64, I32, I32, P]
    lib.oracle_post_reorder.restype = ctypes.c_int
    lib.oracle_post_reorder.argtypes = [P, P, P, I64, I32, I32, P]
    lib.oracle_dense_layer.restype = ctypes.c_int
    lib.oracle_permute_map.restype = ctypes.c_int
    lib.oracle_permute_map.argtypes = [P, I64, I32, I32, I32, I32, I32, I64, P, P, P]
    lib.oracle_dense_layer_map.restype = ctypes.c_int
    lib.oracle_dense_layer_map.argtypes = [P, P, P, I64, I32, I32, I32, I32, I32, I32, I32, I32,
                                           P, P, P, P, I32, P]
    lib.oracle_dense_layer.argtypes = [P, P, P, I64, I32, I32, I32, I32, I32, I32,
                                       P, P, P, P, I32, P]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    lib.oracle_get_threads.argtypes = []
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


# ---- number formats -------------------------------------------------------

def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def e4m3_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)


def bf16_rne(v: float) -> int:
    return int(_load().oracle_bf16_rne(float(v)))


def bf16_rne_f64(v: float) -> int:
    return int(_load().oracle_bf16_rne_f64(float(v)))


def exp_ref(x: float) -> float:
    return float(_load().oracle_exp_ref(float(x)))


def sigmoid(x: float) -> float:
    return float(_load().oracle_sigmoid(float(x)))


def silu_mul_bf16(g: float, u: float) -> int:
    return int(_load().oracle_silu_mul_bf16(float(g), float(u)))


def math_vec(x):
    """exp_ref, sigmoid and the fp32 SiLU x / (1 + exp_ref(-x)) of every fp32 in x."""
    x = _c(np.asarray(x, dtype=np.float32).reshape(-1), np.float32)
    e, sg, sl = (np.empty_like(x) for _ in range(3))
    _check(_load().oracle_math_vec(_p(x), len(x), _p(e), _p(sg), _p(sl)), "math_vec")
    return e, sg, sl


# ---- stages ---------------------------------------------------------------

def select_experts(logits, bias, topk, n_group=1, topk_group=1, score_fn=0, renormalize=1,
                   rsf=1.0, apply_rsf=1, n_shared=0, shared_weight=1.0):
    """Stage 1: returns (ids int32 [T, topk + n_shared], weights fp32 [T, topk + n_shared]).

    Shared experts (this build's reading of the pages' shared-expert fusion):
    every token also takes experts E..E+n_shared-1 with weight shared_weight,
    after its routed slots."""
    if n_shared:
        ids, w = select_experts(logits, bias, topk, n_group, topk_group, score_fn, renormalize,
                                rsf, apply_rsf)
        T, E = np.asarray(logits).shape
        sid = np.broadcast_to(np.arange(E, E + n_shared, dtype=np.int32), (T, n_shared))
        sw = np.full((T, n_shared), shared_weight, dtype=np.float32)
        return np.ascontiguousarray(np.concatenate([ids, sid], 1)), np.ascontiguousarray(np.concatenate([w, sw], 1))
    logits = _c(logits, np.float32)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float32)
    rc = _load().oracle_select_experts(_p(logits), _p(bias), T, E, topk, n_group, topk_group,
                                       score_fn, renormalize, float(rsf), apply_rsf,
                                       _p(ids), _p(w))
    _check(rc, "select_experts")
    return ids, w


def permute(ids, expert_start, num_local, m_cap, shared_base=0, n_shared=0):
    """Stage 2 (indices): returns (src2dst [T*topk], dst2src [m_cap],
    seg_indptr [num_local+n_shared+1]). num_local counts the routed local experts;
    ids in [shared_base, shared_base + n_shared) are local experts num_local.."""
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    src2dst = np.empty(T * topk, dtype=np.int32)
    dst2src = np.empty(max(m_cap, 0), dtype=np.int32)
    seg = np.empty(num_local + n_shared + 1, dtype=np.int32)
    rc = _load().oracle_permute_map(_p(ids), T, topk, expert_start, num_local, shared_base, n_shared,
                                    m_cap, _p(src2dst), _p(dst2src), _p(seg))
    _check(rc, "permute")
    return src2dst, dst2src, seg


def pre_reorder_quant(x_bits, src2dst, topk, act_quant, m_cap):
    """Stage 2 (data): returns (a_q uint8 [m_cap, H], a_scale fp32). Rows never written are 0."""
    x_bits = _c(x_bits, np.uint16)
    src2dst = _c(src2dst, np.int32)
    T, H = x_bits.shape
    G = -(-H // 128)
    a_q = np.zeros((m_cap, H), dtype=np.uint8)
    n_scale = 1 if act_quant == 0 else (m_cap if act_quant == 1 else m_cap * G)
    a_scale = np.zeros(max(n_scale, 1), dtype=np.float32)
    rc = _load().oracle_pre_reorder_quant(_p(x_bits), _p(src2dst), T, H, topk, act_quant,
                                          _p(a_q), _p(a_scale))
    _check(rc, "pre_reorder_quant")
    return a_q, a_scale


def grouped_gemm(a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr, flags=0):
    """Stage 3: returns C bf16 bits [m_cap, N] (rows >= M are 0)."""
    a_q = _c(a_q, np.uint8)
    b_q = _c(b_q, np.uint8)
    a_scale = _c(a_scale, np.float32)
    b_scale = _c(b_scale, np.float32)
    seg = _c(seg_indptr, np.int32)
    m_cap, K = a_q.shape
    num_local, N, K2 = b_q.shape
    assert K == K2
    c = np.zeros((m_cap, N), dtype=np.uint16)
    rc = _load().oracle_grouped_gemm(_p(a_q), _p(a_scale), act_quant, _p(b_q), _p(b_scale),
                                     w_quant, _p(seg), num_local, N, K, _p(c), flags)
    _check(rc, "grouped_gemm")
    return c


def grouped_gemm_rows(a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg_indptr, rows):
    """Stage 3 for selected rows only: returns bf16 bits [len(rows), N]."""
    a_q = _c(a_q, np.uint8)
    b_q = _c(b_q, np.uint8)
    a_scale = _c(a_scale, np.float32)
    b_scale = _c(b_scale, np.float32)
    seg = _c(seg_indptr, np.int32)
    rows = _c(rows, np.int64)
    K = a_q.shape[1]
    num_local, N, K2 = b_q.shape
    assert K == K2
    c = np.zeros((len(rows), N), dtype=np.uint16)
    rc = _load().oracle_grouped_gemm_rows(_p(a_q), _p(a_scale), act_quant, _p(b_q), _p(b_scale),
                                          w_quant, _p(seg), num_local, N, K, _p(rows), len(rows),
                                          _p(c))
    _check(rc, "grouped_gemm_rows")
    return c


def e2m1_value(nibble: int) -> float:
    return float(_load().oracle_e2m1_value(int(nibble)))


def e8m0_value(code: int) -> float:
    return float(_load().oracle_e8m0_value(int(code)))


def _fp4_args(a_q, b_fp4, b_e8m0):
    a_q = _c(a_q, np.uint8)
    b_fp4 = _c(b_fp4, np.uint8)
    b_e8m0 = _c(b_e8m0, np.uint8)
    K = a_q.shape[1]
    num_local, N, Kh = b_fp4.shape
    assert 2 * Kh == K and b_e8m0.shape == (num_local, N, K // 32)
    return a_q, b_fp4, b_e8m0, num_local, N, K


def grouped_gemm_mxfp4(a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant, seg_indptr):
    """Stage 3 with MXFP4 weights (packed codes [E_l, N, K/2], E8M0 [E_l, N, K/32]):
    returns C bf16 bits [m_cap, N] (rows >= M are 0)."""
    a_q, b_fp4, b_e8m0, num_local, N, K = _fp4_args(a_q, b_fp4, b_e8m0)
    a_scale = _c(a_scale, np.float32)
    b_scale = _c(b_scale, np.float32)
    seg = _c(seg_indptr, np.int32)
    c = np.zeros((a_q.shape[0], N), dtype=np.uint16)
    rc = _load().oracle_grouped_gemm_mxfp4(_p(a_q), _p(a_scale), act_quant, _p(b_fp4), _p(b_e8m0),
                                           _p(b_scale), w_quant, _p(seg), num_local, N, K, _p(c))
    _check(rc, "grouped_gemm_mxfp4")
    return c


def grouped_gemm_mxfp4_rows(a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant, seg_indptr, rows):
    """grouped_gemm_mxfp4 for selected rows only: returns bf16 bits [len(rows), N]."""
    a_q, b_fp4, b_e8m0, num_local, N, K = _fp4_args(a_q, b_fp4, b_e8m0)
    a_scale = _c(a_scale, np.float32)
    b_scale = _c(b_scale, np.float32)
    seg = _c(seg_indptr, np.int32)
    rows = _c(rows, np.int64)
    c = np.zeros((len(rows), N), dtype=np.uint16)
    rc = _load().oracle_grouped_gemm_mxfp4_rows(_p(a_q), _p(a_scale), act_quant, _p(b_fp4), _p(b_e8m0),
                                                _p(b_scale), w_quant, _p(seg), num_local, N, K,
                                                _p(rows), len(rows), _p(c))
    _check(rc, "grouped_gemm_mxfp4_rows")
    return c


def act_requant(gateup_bits, seg_indptr, act_quant):
    """Stage 4: returns (a_q uint8 [m_cap, I], a_scale fp32)."""
    gu = _c(gateup_bits, np.uint16)
    seg = _c(seg_indptr, np.int32)
    m_cap, two_i = gu.shape
    I = two_i // 2
    G = -(-I // 128)
    a_q = np.zeros((m_cap, I), dtype=np.uint8)
    n_scale = 1 if act_quant == 0 else (m_cap if act_quant == 1 else m_cap * G)
    a_scale = np.zeros(max(n_scale, 1), dtype=np.float32)
    rc = _load().oracle_act_requant(_p(gu), _p(seg), len(seg) - 1, I, act_quant, _p(a_q),
                                    _p(a_scale))
    _check(rc, "act_requant")
    return a_q, a_scale


def router_logits(x_bits, wg_bits):
    """Router projection: fp32 [T, E] = fp32(sum_h x[t,h] * wg[e,h]) of bf16 x [T, H], wg [E, H]."""
    x = _c(x_bits, np.uint16)
    wg = _c(wg_bits, np.uint16)
    T, H = x.shape
    E, H2 = wg.shape
    assert H == H2
    out = np.empty((T, E), dtype=np.float32)
    rc = _load().oracle_router_logits(_p(x), _p(wg), T, H, E, _p(out))
    _check(rc, "router_logits")
    return out


def post_reorder(down_bits, src2dst, weights, T, topk):
    """Stage 5: returns out bf16 bits [T, H]."""
    down = _c(down_bits, np.uint16)
    src2dst = _c(src2dst, np.int32)
    w = _c(weights, np.float32)
    H = down.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    rc = _load().oracle_post_reorder(_p(down), _p(src2dst), _p(w), T, H, topk, _p(out))
    _check(rc, "post_reorder")
    return out


def dense_layer(x_bits, ids, weights, I, expert_start, num_local, act_quant,
                w13, s13, w2, s2, w_quant, shared_base=0, n_shared=0):
    """Dense per-token layer (no permutation): returns out bf16 bits [T, H]."""
    x_bits = _c(x_bits, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(weights, np.float32)
    T, H = x_bits.shape
    topk = ids.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    rc = _load().oracle_dense_layer_map(_p(x_bits), _p(ids), _p(w), T, H, I, topk, expert_start,
                                        num_local, shared_base, n_shared, act_quant,
                                        _p(_c(w13, np.uint8)), _p(_c(s13, np.float32)),
                                        _p(_c(w2, np.uint8)), _p(_c(s2, np.float32)), w_quant,
                                        _p(out))
    _check(rc, "dense_layer")
    return out


def layer(inp, flags=0):
    """Whole permuted layer on a workloads.LayerInputs; returns a dict of every stage's outputs."""
    cfg = inp.cfg
    ids, w = select_experts(inp.logits, inp.bias, cfg.topk, cfg.n_group, cfg.topk_group,
                            cfg.score_fn, cfg.renormalize, cfg.rsf, cfg.apply_rsf,
                            cfg.n_shared, cfg.shared_weight)
    m_cap = cfg.m_cap
    src2dst, dst2src, seg = permute(ids, cfg.expert_start, cfg.num_local, m_cap, cfg.E, cfg.n_shared)
    a13, s_a13 = pre_reorder_quant(inp.x, src2dst, cfg.slots, cfg.act_quant, m_cap)
    if cfg.w_fp4:
        c13 = grouped_gemm_mxfp4(a13, s_a13, cfg.act_quant, inp.w13, inp.w13_e8m0, inp.w13_scale,
                                 cfg.w_quant, seg)
    else:
        c13 = grouped_gemm(a13, s_a13, cfg.act_quant, inp.w13, inp.w13_scale, cfg.w_quant, seg, flags)
    a2, s_a2 = act_requant(c13, seg, cfg.act_quant)
    if cfg.w_fp4:
        c2 = grouped_gemm_mxfp4(a2, s_a2, cfg.act_quant, inp.w2, inp.w2_e8m0, inp.w2_scale,
                                cfg.w_quant, seg)
    else:
        c2 = grouped_gemm(a2, s_a2, cfg.act_quant, inp.w2, inp.w2_scale, cfg.w_quant, seg, flags)
    out = post_reorder(c2, src2dst, w, cfg.T, cfg.slots)
    return dict(ids=ids, weights=w, src2dst=src2dst, dst2src=dst2src, seg_indptr=seg,
                a13=a13, a13_scale=s_a13, c13=c13, a2=a2, a2_scale=s_a2, c2=c2, out=out)
