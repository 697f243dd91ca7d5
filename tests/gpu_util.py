"""Helpers for the GPU parity tests: upload seeded inputs, run one libmoe stage
through the C ABI (via the Python binding), download the results, and check
guard regions behind every output buffer.

Every output tensor is allocated with a trailing guard region filled with a
sentinel; ``check_guards`` fails if any kernel wrote past its buffer.
"""
import functools

import numpy as np
import torch

import fp8_grouped_gemm_select_amd as moe
import workloads as W

GUARD = 4096  # elements behind every output buffer
SENTINEL = {torch.uint8: 0xA5, torch.int32: -123456789, torch.float32: float("nan"),
            torch.bfloat16: float("nan")}


def dev():
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=1)
def layer_inputs(name, seed=0):
    """Seeded inputs of a named workload, weights included. The last one drawn is
    kept, so consecutive tests of one workload share a single draw of its
    weights (the Mixtral-shaped experts alone are 1.4 GB of codes)."""
    return W.gen_layer_inputs(W.CONFIGS[name], seed=seed)


def up(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev())


def up_bf16(bits):
    return up(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16), torch.bfloat16)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """A tensor of `shape` followed by GUARD sentinel elements."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(int(s) for s in shape)
        n = int(np.prod(shape)) if len(shape) else 1
        self.full = torch.empty(n + GUARD, dtype=dtype, device=dev())
        s = SENTINEL[dtype]
        self.full.fill_(s)
        if fill is not None:
            self.full[:n].fill_(fill)
        self.n = n
        self.t = self.full[:n].view(shape)
        self.dtype = dtype

    def check(self, name="buffer"):
        tail = self.full[self.n:]
        if self.dtype in (torch.float32, torch.bfloat16):
            ok = bool(torch.isnan(tail.float()).all())
        else:
            ok = bool((tail == SENTINEL[self.dtype]).all())
        assert ok, f"{name}: a kernel wrote past the end of the buffer"


def run_select(logits, bias, topk, n_group=1, topk_group=1, score_fn=0, renormalize=1, rsf=1.0,
               apply_rsf=1):
    T = logits.shape[0]
    ids = Guarded((T, topk), torch.int32)
    w = Guarded((T, topk), torch.float32)
    lt = up(logits)
    bt = up(bias) if bias is not None else None
    moe.moe_select_experts(lt, bt, ids.t, w.t, topk=topk, n_group=n_group, topk_group=topk_group,
                           score_fn=score_fn, renormalize=renormalize, routed_scaling_factor=rsf,
                           apply_rsf=apply_rsf)
    torch.cuda.synchronize()
    ids.check("topk_ids")
    w.check("topk_weights")
    return ids.t.cpu().numpy(), w.t.cpu().numpy()


def scale_numel(mode, m_cap, K):
    return 1 if mode == moe.ACT_PER_TENSOR else (m_cap if mode == moe.ACT_PER_TOKEN else m_cap * (-(-K // 128)))


def run_pre(x_bits, ids, expert_start, num_local, act_quant, m_cap=None):
    T, H = x_bits.shape
    topk = ids.shape[1]
    if m_cap is None:
        m_cap = T * min(topk, num_local)
    a_q = Guarded((m_cap, H), torch.uint8)
    a_s = Guarded((scale_numel(act_quant, m_cap, H),), torch.float32)
    s2d = Guarded((T * topk,), torch.int32)
    d2s = Guarded((m_cap,), torch.int32)
    seg = Guarded((num_local + 1,), torch.int32)
    ws = torch.empty(moe.moe_workspace_bytes(T, topk, num_local), dtype=torch.uint8, device=dev())
    moe.moe_pre_reorder_quant(up_bf16(x_bits), up(ids.astype(np.int32)), a_q.t, a_s.t, s2d.t,
                              d2s.t, seg.t, ws, expert_start=expert_start, num_local=num_local,
                              act_quant=act_quant)
    torch.cuda.synchronize()
    for g, n in [(a_q, "a_q"), (a_s, "a_scale"), (s2d, "src2dst"), (d2s, "dst2src"), (seg, "seg")]:
        g.check(n)
    return dict(a_q=a_q.t.cpu().numpy(), a_scale=a_s.t.cpu().numpy(), src2dst=s2d.t.cpu().numpy(),
                dst2src=d2s.t.cpu().numpy(), seg=seg.t.cpu().numpy())


def run_gemm(a_q, a_scale, act_quant, b_q, b_scale, w_quant, seg, b_dev=None):
    m_cap, K = a_q.shape
    N = b_q.shape[1] if b_q is not None else b_dev.shape[1]
    c = Guarded((m_cap, N), torch.bfloat16)
    bt = b_dev if b_dev is not None else up(b_q)
    moe.moe_grouped_gemm_fp8(up(a_q), up(a_scale), bt, up(np.asarray(b_scale).reshape(-1)),
                             up(seg.astype(np.int32)), c.t, act_quant=act_quant, w_quant=w_quant)
    torch.cuda.synchronize()
    c.check("c")
    return bf16_bits(c.t)


def run_act(gu_bits, seg, act_quant):
    m_cap, two_i = gu_bits.shape
    I = two_i // 2
    a_q = Guarded((m_cap, I), torch.uint8)
    a_s = Guarded((scale_numel(act_quant, m_cap, I),), torch.float32)
    ws = torch.empty(moe.moe_workspace_bytes(1, 1, 1), dtype=torch.uint8, device=dev())
    moe.moe_act_requant(up_bf16(gu_bits), up(seg.astype(np.int32)), a_q.t, a_s.t, ws,
                        act_quant=act_quant)
    torch.cuda.synchronize()
    a_q.check("a_q")
    a_s.check("a_scale")
    return a_q.t.cpu().numpy(), a_s.t.cpu().numpy()


def run_post(down_bits, src2dst, weights, T, topk):
    H = down_bits.shape[1]
    out = Guarded((T, H), torch.bfloat16)
    moe.moe_post_reorder(up_bf16(down_bits), up(src2dst.astype(np.int32)),
                         up(weights.astype(np.float32)), out.t)
    torch.cuda.synchronize()
    out.check("out")
    return bf16_bits(out.t)


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close_layer(got_bits, ref_bits, atol=1e-2, rtol=2e-2, what="output"):
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} values outside "
                           f"atol {atol} + rtol {rtol}; worst |diff| {err.max():.4g}")


def assert_within_bf16_ulps(got_bits, ref_bits, ulps=1, what="output"):
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    ulp = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
    err = np.abs(g - r)
    bad = err > ulps * ulp * (1 + 1e-9)
    assert not bad.any(), f"{what}: {int(bad.sum())} values more than {ulps} bf16 ulp away"


def assert_sum_close(got_bits, ref_bits, abs_terms, n_terms, what="output", ulps=1, chunk=128,
                     mfma=True):
    """|got - ref| <= `ulps` bf16 ulps of ref + the summation error of both sides.

    The oracle sums its n_terms exact products sequentially in fp32 (error at
    most n_terms * 2^-24 * sum|terms|). The GPU's FP8 MFMA adds `chunk` products
    per instruction and does not round like a sequence of fp32 additions: its
    internal sum keeps about 14 bits below the largest magnitude it holds (the
    accumulator it adds into included). Each of the ceil(n_terms / chunk)
    instructions is allowed 2^-13 * sum|terms| of error, plus one fp32 rounding
    each. With mfma=False (a plain fp32 loop on the GPU) the GPU side gets the
    sequential-sum bound instead. abs_terms is the sum of the absolute values of
    the summed products.
    Returns the worst observed |got - ref| / sum|terms| (printed by the callers)."""
    g = bf16_to_f64(got_bits)
    r = bf16_to_f64(ref_bits)
    ulp = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
    if mfma:
        nchunks = -(-int(n_terms) // chunk)
        rel = n_terms * 2.0 ** -24 + nchunks * (2.0 ** -13 + 2.0 ** -24)
    else:
        rel = 2 * n_terms * 2.0 ** -24
    bound = ulps * ulp * (1 + 1e-9) + rel * abs_terms
    err = np.abs(g - r)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} values outside the bound; "
                           f"worst excess {(err - bound).max():.3g}")
    same = float((np.asarray(got_bits) == np.asarray(ref_bits)).mean())
    assert same > 0.75, f"{what}: only {same:.3f} of the values are bit-identical"
    excess = np.maximum(err - ulp, 0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(abs_terms > 0, excess / abs_terms, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def fp4_abs_values(packed, e8m0):
    """|value| (fp64) of MXFP4 weights [.., N, K/2] with E8M0 scales [.., N, K/32],
    decoded with the oracle's E2M1 / E8M0 definitions."""
    import oracle
    table = np.array([abs(oracle.e2m1_value(c)) for c in range(16)])
    packed = np.asarray(packed)
    nib = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    nib[..., 0::2], nib[..., 1::2] = packed & 15, packed >> 4
    scale = np.ldexp(1.0, np.asarray(e8m0).astype(np.int64) - 127)
    return table[nib] * np.repeat(scale, 32, axis=-1)


def run_gemm_fp4(a_q, a_scale, act_quant, b_fp4, b_e8m0, b_scale, w_quant, seg):
    m_cap, K = a_q.shape
    N = b_fp4.shape[1]
    c = Guarded((m_cap, N), torch.bfloat16)
    moe.moe_grouped_gemm_mxfp4(up(a_q), up(a_scale), up(b_fp4), up(b_e8m0),
                               up(np.asarray(b_scale, np.float32).reshape(-1)), up(seg.astype(np.int32)),
                               c.t, act_quant=act_quant, w_quant=w_quant)
    torch.cuda.synchronize()
    c.check("c")
    return bf16_bits(c.t)
