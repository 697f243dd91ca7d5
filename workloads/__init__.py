"""Seeded synthetic workloads for the EP-MoE FP8 layer.

This module only draws random numbers and casts them to storage types (bf16,
OCP e4m3fn through torch's own dtype conversion). It holds none of the layer's
arithmetic: no routing, permutation, activation quantisation, GEMM or combine.
Both the CPU oracle and the HIP library consume what it returns.

Shapes follow the five workloads the MoE layer is studied on: a tiny layer, a
DeepSeek-V3-shaped layer's one-GPU expert-parallel share at decode (T=128) and
prefill (T=8192), a Mixtral-shaped layer with every expert local, and a skewed
128-expert layer with block scales.

Every tensor comes from ``numpy.random.default_rng([seed, tensor_id, ...])``
with tensor_id 0 = tokens X, 1 = router weights W_g, 2 = correction bias,
3 = w13, 4 = w2, 5 = routing skew. Expert weights are drawn per expert
(``[seed, 3, e]``), so one expert's weights can be regenerated on their own.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np
import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

ACT_PER_TENSOR = 0
ACT_PER_TOKEN = 1
ACT_PER_GROUP = 2

W_PER_EXPERT = 0
W_PER_CHANNEL = 1
W_BLOCK = 2

E4M3_MAX = 448.0
QBLOCK = 128

TID_X, TID_WG, TID_BIAS, TID_W13, TID_W2, TID_SKEW = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One MoE layer workload (shapes, routing and quantisation modes)."""
    name: str
    T: int                 # tokens
    H: int                 # hidden size (K of w13, N of w2)
    I: int                 # moe intermediate size (w13 has N = 2I, w2 has K = I)
    E: int                 # routed experts in the whole layer
    topk: int
    num_local: int         # experts held by this GPU
    expert_start: int = 0  # first local expert id
    score_fn: int = SCORE_SOFTMAX
    n_group: int = 1
    topk_group: int = 1
    renormalize: int = 1
    rsf: float = 1.0       # routed_scaling_factor
    apply_rsf: int = 1
    use_bias: bool = False
    act_quant: int = ACT_PER_TOKEN
    w_quant: int = W_PER_EXPERT
    zipf_skew: float = 0.0  # > 0: router logits biased so expert popularity follows Zipf(s)
    cold_experts: int = 0   # experts never drawn by the skew
    n_shared: int = 0       # shared experts: ids E.., taken by every token, local after the routed
    shared_weight: float = 1.0
    w_fp4: bool = False     # expert weights as MXFP4 codes + E8M0 block scales (w_quant: the fp32 factor)
    description: str = ""

    @property
    def slots(self) -> int:
        """Slots per token: the top-k routed ones plus the shared experts."""
        return self.topk + self.n_shared

    @property
    def local_experts(self) -> int:
        """Experts whose weights this GPU holds: routed local + shared."""
        return self.num_local + self.n_shared

    @property
    def m_cap(self) -> int:
        """Upper bound on local (token, slot) pairs: T * min(slots, local experts)."""
        return self.T * min(self.slots, self.local_experts)

    def with_tokens(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=T)


CONFIGS = {
    "tiny": MoEConfig(
        name="tiny", T=16, H=128, I=64, E=8, topk=2, num_local=8,
        score_fn=SCORE_SOFTMAX, rsf=1.0, act_quant=ACT_PER_TOKEN, w_quant=W_PER_EXPERT,
        description="T=16, H=128, I=64, E=8 top-2 softmax, per-expert weight scale, "
                    "per-token activations"),
    "dsv3_decode_ep": MoEConfig(
        name="dsv3_decode_ep", T=128, H=7168, I=2048, E=256, topk=8, num_local=32,
        expert_start=0, score_fn=SCORE_SIGMOID, n_group=8, topk_group=4, rsf=2.5,
        use_bias=True, act_quant=ACT_PER_TOKEN, w_quant=W_PER_CHANNEL,
        description="DeepSeek-V3 shape, one GPU's EP share (32 of 256 experts), decode T=128"),
    "dsv3_prefill_ep": MoEConfig(
        name="dsv3_prefill_ep", T=8192, H=7168, I=2048, E=256, topk=8, num_local=32,
        expert_start=0, score_fn=SCORE_SIGMOID, n_group=8, topk_group=4, rsf=2.5,
        use_bias=True, act_quant=ACT_PER_TOKEN, w_quant=W_PER_CHANNEL,
        description="DeepSeek-V3 shape, one GPU's EP share (32 of 256 experts), prefill T=8192"),
    "mixtral": MoEConfig(
        name="mixtral", T=4096, H=4096, I=14336, E=8, topk=2, num_local=8,
        score_fn=SCORE_SOFTMAX, rsf=1.0, act_quant=ACT_PER_TENSOR, w_quant=W_PER_EXPERT,
        description="Mixtral shape, all 8 experts local, T=4096, per-tensor activation scale"),
    "skewed_block": MoEConfig(
        name="skewed_block", T=16384, H=2048, I=768, E=128, topk=8, num_local=128,
        score_fn=SCORE_SOFTMAX, rsf=1.0, act_quant=ACT_PER_GROUP, w_quant=W_BLOCK,
        zipf_skew=1.2, cold_experts=4,
        description="128 experts all local, Zipf(1.2) popularity with 4 cold experts, "
                    "T=16384, 128x128 weight blocks and 1x128 activation groups"),
}

# Extension workloads (not in CONFIG_ORDER): the DeepSeek-V3 shares with the one
# shared expert (intermediate 2048, weight 1 next to the rsf-scaled routed ones)
# fused into the same grouped GEMMs.
CONFIGS["dsv3_decode_ep_shared"] = dataclasses.replace(
    CONFIGS["dsv3_decode_ep"], name="dsv3_decode_ep_shared", n_shared=1, shared_weight=1.0,
    description="dsv3_decode_ep plus one shared expert (weight 1) fused as local expert 32")
CONFIGS["dsv3_prefill_ep_shared"] = dataclasses.replace(
    CONFIGS["dsv3_prefill_ep"], name="dsv3_prefill_ep_shared", n_shared=1, shared_weight=1.0,
    description="dsv3_prefill_ep plus one shared expert (weight 1) fused as local expert 32")

# FP4-weight extension workloads: the same DeepSeek-V3 shares with MXFP4 expert
# weights (E2M1 codes, one E8M0 scale per 32 input elements, and a per-expert
# fp32 factor).
CONFIGS["dsv3_decode_ep_fp4"] = dataclasses.replace(
    CONFIGS["dsv3_decode_ep"], name="dsv3_decode_ep_fp4", w_fp4=True, w_quant=W_PER_EXPERT,
    description="dsv3_decode_ep with MXFP4 expert weights")
CONFIGS["dsv3_prefill_ep_fp4"] = dataclasses.replace(
    CONFIGS["dsv3_prefill_ep"], name="dsv3_prefill_ep_fp4", w_fp4=True, w_quant=W_PER_EXPERT,
    description="dsv3_prefill_ep with MXFP4 expert weights")

CONFIG_ORDER = ["tiny", "dsv3_decode_ep", "dsv3_prefill_ep", "mixtral", "skewed_block"]


def rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([seed, *ids])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even cast), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes through torch's float8_e4m3fn cast (clipped to +-448 first)."""
    t = torch.from_numpy(np.clip(np.ascontiguousarray(a, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def gen_tokens(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """X: bf16(N(0,1)) of shape [T, H], as uint16 bits."""
    x = rng(seed, TID_X).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return to_bf16_bits(x)


def gen_router(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """W_g ~ N(0, 0.02), shape [H, E], fp32."""
    return (rng(seed, TID_WG).standard_normal((cfg.H, cfg.E), dtype=np.float32)
            * np.float32(0.02))


def gen_router_bf16(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """The router weight W_g of gen_router rounded to bf16 and stored one row per
    expert: uint16 bits of shape [E, H] (the layout the GPU router reads)."""
    return np.ascontiguousarray(to_bf16_bits(gen_router(cfg, seed)).T)


def gen_bias(cfg: MoEConfig, seed: int = 0) -> Optional[np.ndarray]:
    """Per-expert correction bias ~ N(0, 0.01) [E], or None when the workload has none."""
    if not cfg.use_bias:
        return None
    return rng(seed, TID_BIAS).standard_normal(cfg.E, dtype=np.float32) * np.float32(0.01)


def zipf_skew_offsets(cfg: MoEConfig, seed: int = 0) -> np.ndarray:
    """[T, E] logit offsets that make expert popularity follow Zipf(s).

    Experts are ranked by a seeded permutation; the ``cold_experts`` lowest-ranked
    never get drawn. For every token, ``topk`` distinct warm experts are drawn
    without replacement with probability proportional to rank**-s (Gumbel top-k,
    which is the same distribution as successive draws without replacement), and
    +8.0 is added to their logits. +8 is far above the ~N(0, 0.9^2) projection
    noise, so top-k routing returns exactly the drawn set.
    """
    g = rng(seed, TID_SKEW)
    order = g.permutation(cfg.E)                 # order[r] = expert at rank r (rank 0 hottest)
    warm = cfg.E - cfg.cold_experts
    ranks = np.arange(1, warm + 1, dtype=np.float64)
    logw = -cfg.zipf_skew * np.log(ranks)
    gumbel = -np.log(-np.log(g.random((cfg.T, warm))))
    pick = np.argpartition(-(logw[None, :] + gumbel), cfg.topk - 1, axis=1)[:, :cfg.topk]
    off = np.zeros((cfg.T, cfg.E), dtype=np.float32)
    rows = np.repeat(np.arange(cfg.T), cfg.topk)
    off[rows, order[pick.reshape(-1)]] = np.float32(8.0)
    return off


def gen_logits(cfg: MoEConfig, x_bits: np.ndarray, seed: int = 0) -> np.ndarray:
    """Router logits fp32 [T, E] = fp32(X) @ W_g (computed once on the CPU), plus skew."""
    wg = gen_router(cfg, seed)
    logits = bf16_bits_to_f32(x_bits) @ wg
    if cfg.zipf_skew > 0:
        logits = logits + zipf_skew_offsets(cfg, seed)
    return np.ascontiguousarray(logits, dtype=np.float32)


def _weight_scales(w: np.ndarray, mode: int) -> np.ndarray:
    """amax / 448 at the requested granularity for one expert's [N, K] matrix."""
    a = np.abs(w)
    if mode == W_PER_EXPERT:
        amax = np.array([a.max()], dtype=np.float32)
    elif mode == W_PER_CHANNEL:
        amax = a.max(axis=1).astype(np.float32)
    elif mode == W_BLOCK:
        N, K = w.shape
        nb, kb = -(-N // QBLOCK), -(-K // QBLOCK)
        pad = np.zeros((nb * QBLOCK, kb * QBLOCK), dtype=np.float32)
        pad[:N, :K] = a
        amax = pad.reshape(nb, QBLOCK, kb, QBLOCK).max(axis=(1, 3)).astype(np.float32)
    else:
        raise ValueError(mode)
    amax = np.maximum(amax, np.float32(1e-10))
    return (amax / np.float32(E4M3_MAX)).astype(np.float32)


def _expand_scales(s: np.ndarray, mode: int, N: int, K: int) -> np.ndarray:
    if mode == W_PER_EXPERT:
        return np.full((N, K), s[0], dtype=np.float32)
    if mode == W_PER_CHANNEL:
        return np.repeat(s[:, None], K, axis=1)
    full = np.repeat(np.repeat(s, QBLOCK, axis=0), QBLOCK, axis=1)
    return np.ascontiguousarray(full[:N, :K])


def gen_expert_weight(cfg: MoEConfig, which: str, e_local: int, seed: int = 0):
    """One local expert's weight as (codes uint8 [N, K], scales fp32).

    which = "w13": N = 2I (gate rows then up rows), K = H.
    which = "w2":  N = H, K = I.
    Storage is [N, K] (output x input, K contiguous). The workload text lists the
    same weights as [E, K, N]; only the storage order differs.
    Scales: per expert [1], per output channel [N], or 128x128 blocks [N/128, K/128].
    """
    if which == "w13":
        N, K, tid = 2 * cfg.I, cfg.H, TID_W13
    elif which == "w2":
        N, K, tid = cfg.H, cfg.I, TID_W2
    else:
        raise ValueError(which)
    e_global = cfg.expert_start + e_local
    w = rng(seed, tid, e_global).standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    s = _weight_scales(w, cfg.w_quant)
    codes = to_e4m3_codes(w / _expand_scales(s, cfg.w_quant, N, K))
    return codes, s


# Magnitude ranks 0..7 of E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) are drawn
# with probabilities 10, 11, 10, 7, 5, 4, 2, 1 in 50 (a bell shape, like
# block-quantised Gaussian weights), by indexing this table with a uniform byte.
FP4_RANK_TABLE = np.repeat(np.arange(8, dtype=np.uint8), [10, 11, 10, 7, 5, 4, 2, 1])
FP4_E8M0_BASE = 120  # block scales 2^(119..121 - 127)


def gen_expert_weight_fp4(cfg: MoEConfig, which: str, e_local: int, seed: int = 0):
    """One local expert's MXFP4 weight: packed codes uint8 [N, K/2] (element k in
    byte k/2, low nibble for even k), E8M0 block scales uint8 [N, K/32], and the
    fp32 per-expert factor [1] (or per channel [N] under W_PER_CHANNEL).
    Codes and scales are drawn directly: nothing is quantised here."""
    if which == "w13":
        N, K, tid = 2 * cfg.I, cfg.H, TID_W13
    elif which == "w2":
        N, K, tid = cfg.H, cfg.I, TID_W2
    else:
        raise ValueError(which)
    g = rng(seed, tid, cfg.expert_start + e_local, 4)
    rank = FP4_RANK_TABLE[g.integers(0, len(FP4_RANK_TABLE), size=(N, K), dtype=np.uint8)]
    sign = g.integers(0, 2, size=(N, K), dtype=np.uint8)
    nib = rank | (sign << 3)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    e8m0 = (FP4_E8M0_BASE + g.integers(-1, 2, size=(N, K // 32))).astype(np.uint8)
    n_f = 1 if cfg.w_quant == W_PER_EXPERT else N
    factor = g.uniform(0.75, 1.25, size=n_f).astype(np.float32)
    return packed, e8m0, factor


def gen_weights_fp4(cfg: MoEConfig, which: str, seed: int = 0):
    """All local experts: packed [E_l, N, K/2], e8m0 [E_l, N, K/32], factors [E_l, 1 or N]."""
    import concurrent.futures as cf
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(lambda e: gen_expert_weight_fp4(cfg, which, e, seed), range(cfg.local_experts)))
    return (np.stack([p for p, _, _ in parts]), np.stack([s for _, s, _ in parts]),
            np.stack([f for _, _, f in parts]))


def gen_weights(cfg: MoEConfig, which: str, seed: int = 0):
    """All local experts' codes [E_l, N, K] uint8 and scales fp32 (mode-shaped, flattened per expert).

    Experts are drawn in parallel threads; each has its own generator, so the
    result does not depend on the thread count."""
    import concurrent.futures as cf
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(lambda e: gen_expert_weight(cfg, which, e, seed), range(cfg.local_experts)))
    return np.stack([c for c, _ in parts]), np.stack([s.reshape(-1) for _, s in parts])


@dataclasses.dataclass
class LayerInputs:
    cfg: MoEConfig
    x: np.ndarray           # uint16 bf16 bits [T, H]
    logits: np.ndarray      # fp32 [T, E]
    bias: Optional[np.ndarray]
    w13: np.ndarray         # uint8 [E_l, 2I, H]
    w13_scale: np.ndarray   # fp32 [E_l, ...]
    w2: np.ndarray          # uint8 [E_l, H, I]
    w2_scale: np.ndarray
    w13_e8m0: Optional[np.ndarray] = None  # MXFP4 weights only: w13 / w2 are then packed
    w2_e8m0: Optional[np.ndarray] = None   # [E_l, N, K/2] and these the [E_l, N, K/32] scales


def gen_layer_inputs(cfg: MoEConfig, seed: int = 0, weights: bool = True) -> LayerInputs:
    x = gen_tokens(cfg, seed)
    logits = gen_logits(cfg, x, seed)
    bias = gen_bias(cfg, seed)
    e13 = e2 = None
    if weights and cfg.w_fp4:
        w13, e13, s13 = gen_weights_fp4(cfg, "w13", seed)
        w2, e2, s2 = gen_weights_fp4(cfg, "w2", seed)
    elif weights:
        w13, s13 = gen_weights(cfg, "w13", seed)
        w2, s2 = gen_weights(cfg, "w2", seed)
    else:
        w13 = s13 = w2 = s2 = None
    return LayerInputs(cfg, x, logits, bias, w13, s13, w2, s2, e13, e2)


def a_scale_numel(mode: int, m_cap: int, K: int) -> int:
    """Number of activation scales a mode needs: 1, m_cap, or m_cap * ceil(K/128)."""
    if mode == ACT_PER_TENSOR:
        return 1
    if mode == ACT_PER_TOKEN:
        return m_cap
    return m_cap * (-(-K // QBLOCK))


def b_scale_numel(mode: int, num_local: int, N: int, K: int) -> int:
    if mode == W_PER_EXPERT:
        return num_local
    if mode == W_PER_CHANNEL:
        return num_local * N
    return num_local * (-(-N // QBLOCK)) * (-(-K // QBLOCK))
