"""The C-ABI library loads on the host, exports every symbol the header
declares, and rejects bad arguments on the host before enqueueing anything.

These calls never reach the GPU: each one fails a host-side check first (no
compute call runs here), so they run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

import fp8_grouped_gemm_select_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: checks fail before any use


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_header_declares_the_five_stages():
    names = header_functions()
    for n in ["moe_select_experts", "moe_pre_reorder_quant", "moe_grouped_gemm_fp8",
              "moe_act_requant", "moe_post_reorder"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(moe.EXPORTS) == header_functions()


def test_status_strings(lib):
    for code in range(0, -7, -1):
        s = moe.status_string(code)
        assert s.startswith("MOE_")
    assert "unknown" in moe.status_string(5)


def test_workspace_bytes_monotone(lib):
    a = moe.moe_workspace_bytes(128, 8, 32)
    b = moe.moe_workspace_bytes(8192, 8, 32)
    assert 0 < a <= b
    assert moe.moe_workspace_bytes(0, 8, 0) > 0


def test_select_experts_rejects(lib):
    f = lib.moe_select_experts
    def call(T=4, E=8, k=2, ng=1, tg=1, sf=0, bias=None, logits=FAKE):
        return f(logits, bias, T, E, k, ng, tg, sf, 1, 1.0, 1, FAKE, FAKE, None)
    assert call(E=0) == moe.MOE_ERR_INVALID_ARG
    assert call(k=9) == moe.MOE_ERR_UNSUPPORTED            # topk > E
    assert call(E=1024, k=2) == moe.MOE_ERR_UNSUPPORTED    # E > 512
    assert call(k=40, E=64) == moe.MOE_ERR_UNSUPPORTED     # topk > 32
    assert call(ng=3, sf=1) == moe.MOE_ERR_INVALID_ARG     # E % n_group
    assert call(ng=4, tg=1, k=4, sf=1) == moe.MOE_ERR_INVALID_ARG  # one group of 2 < topk
    assert call(ng=4, tg=5, sf=1) == moe.MOE_ERR_INVALID_ARG
    assert call(ng=2, tg=1, sf=0) == moe.MOE_ERR_UNSUPPORTED      # grouped softmax
    assert call(bias=FAKE, sf=0) == moe.MOE_ERR_UNSUPPORTED       # bias with softmax
    assert call(sf=7) == moe.MOE_ERR_INVALID_ARG
    assert call(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(logits=None) == moe.MOE_ERR_NULL
    assert call(logits=ctypes.c_void_p(0x10004)) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert call(T=0) == moe.MOE_OK                                 # empty: nothing to do


def _pre(lib, T=16, H=128, topk=2, num_local=8, act=1, m_cap=32, n_scale=32, ws=FAKE,
         ws_bytes=1 << 20, x=FAKE, seg=FAKE):
    return lib.moe_pre_reorder_quant(x, FAKE, T, H, topk, 0, num_local, act, m_cap, FAKE, FAKE,
                                     n_scale, FAKE, FAKE, seg, ws, ws_bytes, None)


def test_pre_reorder_rejects(lib):
    assert _pre(lib, n_scale=8) == moe.MOE_ERR_SHAPE              # per-token needs m_cap scales
    assert _pre(lib, act=0, n_scale=32) == moe.MOE_ERR_SHAPE      # per-tensor needs exactly 1
    assert _pre(lib, act=2, H=256, n_scale=32) == moe.MOE_ERR_SHAPE  # per-group needs m_cap*H/128
    assert _pre(lib, m_cap=31, n_scale=31) == moe.MOE_ERR_SHAPE   # m_cap < T*min(topk,num_local)
    assert _pre(lib, H=120) == moe.MOE_ERR_UNSUPPORTED            # H % 16
    assert _pre(lib, act=5) == moe.MOE_ERR_INVALID_ARG
    assert _pre(lib, ws=None) == moe.MOE_ERR_WORKSPACE
    assert _pre(lib, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _pre(lib, seg=None) == moe.MOE_ERR_NULL
    assert _pre(lib, x=None) == moe.MOE_ERR_NULL
    assert _pre(lib, x=ctypes.c_void_p(0x10002)) == moe.MOE_ERR_INVALID_ARG


def test_pre_reorder_noalloc_rejects_before_touching_the_device(lib):
    """The allocation-free stage 2 refuses shapes whose scratch exceeds its static
    array (and bad sizes) before any HIP call: these run without a GPU."""
    f = lib.moe_pre_reorder_quant_noalloc
    def call(T=16, topk=2, num_local=8):
        return f(FAKE, FAKE, T, 128, topk, 0, num_local, 1, T * 2, FAKE, FAKE, T * 2, FAKE, FAKE,
                 FAKE, None)
    assert call(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(topk=0) == moe.MOE_ERR_INVALID_ARG
    assert call(num_local=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(topk=33) == moe.MOE_ERR_UNSUPPORTED
    # 1M tokens x 8 slots in chunks of 64, 256 local experts: ~256 MB of counts
    assert call(T=1 << 20, topk=8, num_local=256) == moe.MOE_ERR_WORKSPACE
    # the largest stage-2 scratch among the five workloads fits
    assert moe.moe_workspace_bytes(16384, 8, 128) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == moe.MOE_NOALLOC_SCRATCH_BYTES


def _gemm(lib, act=1, w=0, a_n=64, b_n=4, m_cap=64, N=128, K=256, num_local=4, seg=FAKE, c=FAKE):
    return lib.moe_grouped_gemm_fp8(FAKE, FAKE, a_n, act, FAKE, FAKE, b_n, w, seg, num_local,
                                    m_cap, N, K, c, None)


def test_grouped_gemm_rejects_scale_shapes(lib):
    # The per-token scale must have one entry per row; an expert-sized buffer
    # would be read out of bounds by the row indexing, so it is refused.
    assert _gemm(lib, act=1, a_n=4) == moe.MOE_ERR_SHAPE
    assert _gemm(lib, act=0, a_n=4) == moe.MOE_ERR_SHAPE
    assert _gemm(lib, act=2, a_n=64) == moe.MOE_ERR_SHAPE         # needs 64 * 2
    assert _gemm(lib, w=1, b_n=4) == moe.MOE_ERR_SHAPE            # per channel needs 4*128
    assert _gemm(lib, w=2, b_n=4) == moe.MOE_ERR_SHAPE            # block needs 4*1*2
    assert _gemm(lib, K=100) == moe.MOE_ERR_UNSUPPORTED
    assert _gemm(lib, num_local=2000, b_n=2000) == moe.MOE_ERR_UNSUPPORTED
    assert _gemm(lib, w=7) == moe.MOE_ERR_INVALID_ARG
    assert _gemm(lib, seg=None) == moe.MOE_ERR_NULL
    assert _gemm(lib, c=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG
    assert _gemm(lib, num_local=0, b_n=0) == moe.MOE_OK           # no experts: nothing to do


def test_act_requant_rejects(lib):
    f = lib.moe_act_requant
    assert f(FAKE, FAKE, 4, 64, 64, 1, FAKE, FAKE, 8, FAKE, 1 << 20, None) == moe.MOE_ERR_SHAPE
    assert f(FAKE, FAKE, 4, 64, 64, 0, FAKE, FAKE, 1, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, FAKE, 4, 64, 60, 1, FAKE, FAKE, 64, FAKE, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(FAKE, None, 4, 64, 64, 1, FAKE, FAKE, 64, FAKE, 1 << 20, None) == moe.MOE_ERR_NULL
    assert f(FAKE, FAKE, 4, 64, 64, 9, FAKE, FAKE, 64, FAKE, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG


def test_post_reorder_rejects(lib):
    f = lib.moe_post_reorder
    assert f(FAKE, FAKE, FAKE, 4, 100, 2, 8, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(FAKE, None, FAKE, 4, 128, 2, 8, FAKE, None) == moe.MOE_ERR_NULL
    assert f(FAKE, FAKE, FAKE, -1, 128, 2, 8, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, 0, 128, 2, 8, FAKE, None) == moe.MOE_OK


def test_binding_requires_gpu_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.moe_post_reorder(torch.zeros((4, 16), dtype=torch.bfloat16),
                             torch.zeros(8, dtype=torch.int32), torch.zeros((4, 2)),
                             torch.zeros((4, 16), dtype=torch.bfloat16))


def test_binding_keyword_only():
    import inspect
    sig = inspect.signature(moe.moe_grouped_gemm_fp8)
    assert sig.parameters["act_quant"].kind == inspect.Parameter.KEYWORD_ONLY
    sig = inspect.signature(moe.moe_select_experts)
    assert sig.parameters["topk"].kind == inspect.Parameter.KEYWORD_ONLY


def test_router_select_rejects(lib):
    f = lib.moe_router_select
    def call(T=4, H=64, E=8, k=2, ng=1, tg=1, sf=0, x=FAKE, wg=FAKE, logits=FAKE, ids=FAKE, ws=None,
             ws_bytes=0):
        return f(x, wg, None, T, H, E, k, ng, tg, sf, 1, 1.0, 1, logits, ids, FAKE, ws, ws_bytes, None)
    assert call(H=12) == moe.MOE_ERR_UNSUPPORTED          # H % 8
    assert call(E=6) == moe.MOE_ERR_UNSUPPORTED           # E % 4
    assert call(E=0) == moe.MOE_ERR_INVALID_ARG
    assert call(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(x=None) == moe.MOE_ERR_NULL
    assert call(wg=None) == moe.MOE_ERR_NULL
    assert call(logits=None) == moe.MOE_ERR_NULL
    assert call(x=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG   # misaligned
    assert call(k=9) == moe.MOE_ERR_UNSUPPORTED           # stage-1 limits, checked first
    assert call(ng=3, sf=1) == moe.MOE_ERR_INVALID_ARG
    assert call(ids=None) == moe.MOE_ERR_NULL
    assert call(T=0) == moe.MOE_OK
    # split-K shapes (H % 64 == 0, E % 64 == 0) need the workspace
    need = lib.moe_router_workspace_bytes(4, 128, 64)
    assert need == 4 * 64 * 4 * 2          # two K splits of [T, E] fp32 partials
    assert call(H=128, E=64) == moe.MOE_ERR_WORKSPACE
    assert call(H=128, E=64, ws=FAKE, ws_bytes=need - 4) == moe.MOE_ERR_WORKSPACE
    assert call(H=128, E=64, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == moe.MOE_ERR_INVALID_ARG


def test_router_workspace_sizes(lib):
    f = lib.moe_router_workspace_bytes
    assert f(8192, 7168, 256) == 4 * 8192 * 256 * 4     # 64 tiles x 4 splits fill 256 CUs
    assert f(128, 7168, 256) == 16 * 128 * 256 * 4     # one tile: 16 splits of 7 steps
    assert f(16, 120, 64) == 0                          # H % 64: the unsplit kernel
    assert f(16, 128, 8) == 0                           # E % 64: the unsplit kernel
    assert f(0, 128, 64) == 0


def test_shared_entry_points_reject(lib):
    sel = lib.moe_select_experts_shared
    def s(ns=1, k=2, E=8):
        return sel(FAKE, None, 4, E, k, 1, 1, 0, 1, 1.0, 1, ns, 1.0, FAKE, FAKE, None)
    assert s(ns=-1) == moe.MOE_ERR_INVALID_ARG
    assert s(ns=63, k=2) == moe.MOE_ERR_UNSUPPORTED        # topk + n_shared > 64
    pre = lib.moe_pre_reorder_quant_shared
    def p(start=0, nr=8, base=8, ns=1, m_cap=36, nsc=36):
        return pre(FAKE, FAKE, 4, 128, 9, start, nr, base, ns, 1, m_cap, FAKE, FAKE, nsc, FAKE, FAKE,
                   FAKE, FAKE, 1 << 20, None)
    assert p(base=4) == moe.MOE_ERR_INVALID_ARG             # shared ids inside the routed range
    assert p(ns=65) == moe.MOE_ERR_INVALID_ARG
    assert p(ns=-1) == moe.MOE_ERR_INVALID_ARG
    assert p(m_cap=35, nsc=35) == moe.MOE_ERR_SHAPE         # m_cap < T * min(9, 9)


def test_mxfp4_gemm_rejects(lib):
    f = lib.moe_grouped_gemm_mxfp4
    def call(act=1, w=0, a_n=64, b_n=4, m_cap=64, N=128, K=256, num_local=4, seg=FAKE, c=FAKE, e8=FAKE):
        return f(FAKE, FAKE, a_n, act, FAKE, e8, FAKE, b_n, w, seg, num_local, m_cap, N, K, c, None)
    assert call(act=1, a_n=4) == moe.MOE_ERR_SHAPE
    assert call(w=1, b_n=4) == moe.MOE_ERR_SHAPE                 # per channel needs 4*128
    assert call(act=2, a_n=128) == moe.MOE_ERR_UNSUPPORTED       # per-group activations
    assert call(w=2) == moe.MOE_ERR_UNSUPPORTED                  # block fp32 weight scales
    assert call(K=192) == moe.MOE_ERR_UNSUPPORTED                # K % 128
    assert call(N=120) == moe.MOE_ERR_UNSUPPORTED
    assert call(w=7) == moe.MOE_ERR_INVALID_ARG
    assert call(seg=None) == moe.MOE_ERR_NULL
    assert call(e8=None) == moe.MOE_ERR_NULL
    assert call(e8=ctypes.c_void_p(0x10002)) == moe.MOE_ERR_INVALID_ARG  # scales need 4-byte alignment
    assert call(c=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG
    assert call(num_local=0, b_n=0) == moe.MOE_OK
