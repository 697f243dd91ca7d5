#!/usr/bin/env python3
"""Benchmark: one EP-MoE layer forward (all five stages) on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens:
select_experts -> pre_reorder_quant -> grouped GEMM (w13) -> act_requant ->
grouped GEMM (w2) -> post_reorder, enqueued on one stream. Inputs and weights
are resident in HBM before the timed region. The default workload is the
DeepSeek-V3-shaped prefill share of one GPU in an 8-way expert-parallel layer
(T=8192 tokens, 32 of 256 experts local), the configuration the grouped-GEMM
target is stated for.

Prints one JSON line: whole-job tokens/s of the layer pass replayed from a HIP
graph (captured once; the timed steps are replays, so the gaps between the
eight kernel launches of a pass are not paid from the host), the eager pass's
tokens/s beside it, the dominant kernel's roofline figures (HIP events around
every launch inside the eager timed region) and the CPU oracle's tokens/s on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "EP-MoE layer tokens/s at 1 GPU; grouped FP8 GEMM TFLOP/s as % of MFMA peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3_prefill_ep")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the separately timed extension rows (router projection, FP4 layer) "
                        "and the decode-share layer")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens in the oracle's timed sample (0: per-workload default)")
    p.add_argument("--no-graph", action="store_true",
                   help="time the headline from eager passes only (no HIP graph; for counter runs)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the on-box ceilings (streaming copy and read, FP8 MFMA loop)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after the run, copy this many MiB once (a plain copy kernel for counter calibration)")
    return p.parse_args()


def algorithmic_work(cfg, seg, a_scale_bytes13, a_scale_bytes2, w13_scale_numel, w2_scale_numel,
                     tokens_local=None):
    """Bytes each stage must move (inputs read once, outputs written once) and GEMM FLOPs.
    Weights of experts with rows: e4m3 codes (1 byte each) or MXFP4 (half a byte
    each plus one E8M0 byte per 32), and their fp32 scales. Stage 2 reads the x
    rows of the `tokens_local` tokens that have a local pair (all T when not
    given), plus all of x once more for the per-tensor amax."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.slots
    M = int(seg[-1])
    counts = np.diff(seg)
    nonempty = int((counts > 0).sum())
    El = cfg.local_experts
    per_w = (0.5 + 1.0 / 32) if cfg.w_fp4 else 1.0
    b13 = int(nonempty * 2 * I * H * per_w) + w13_scale_numel * 4 * nonempty // max(El, 1)
    b2 = int(nonempty * H * I * per_w) + w2_scale_numel * 4 * nonempty // max(El, 1)
    tok_local = T if tokens_local is None else int(tokens_local)
    work = {}
    work["select"] = dict(bytes=T * E * 4 + (E * 4 if cfg.use_bias else 0) + T * k * 8, flops=0)
    # pre_reorder: ids + x rows of tokens with a local pair (+ a second read of x for the
    # per-tensor amax), codes + scales of M rows, src2dst / dst2src / seg
    work["pre_reorder"] = dict(bytes=T * k * 4 + tok_local * H * 2 + (T * H * 2 if cfg.act_quant == 0 else 0)
                               + M * H + a_scale_bytes13 + T * k * 4 + cfg.m_cap * 4 + (El + 1) * 4,
                               flops=0)
    work["gemm_w13"] = dict(bytes=M * H + a_scale_bytes13 + b13 + M * 2 * I * 2 + (El + 1) * 4,
                            flops=2 * M * (2 * I) * H)
    work["act_requant"] = dict(bytes=M * 2 * I * 2 * (2 if cfg.act_quant == 0 else 1) + M * I
                               + a_scale_bytes2, flops=0)
    work["gemm_w2"] = dict(bytes=M * I + a_scale_bytes2 + b2 + M * H * 2 + (El + 1) * 4,
                           flops=2 * M * H * I)
    work["post_reorder"] = dict(bytes=M * H * 2 + T * k * 8 + T * H * 2, flops=0)
    return work, M, nonempty


STAGES = ["select", "pre_reorder", "gemm_w13", "act_requant", "gemm_w2", "post_reorder"]


def time_layer(cfg, inp, steps, warmup, moe, torch, dev, graph=False):
    """Upload one workload's inputs, run `warmup` untimed layer passes, then time
    exactly `steps` passes (wall clock between synchronisations) with HIP events
    between the stages on the launch stream. Returns (ms per step, mean ms per
    stage, the layer buffers, the two weight-scale tensors). With graph=True the
    pass is captured once in a HIP graph and the timed steps are replays
    (per-stage times are then None)."""
    def up(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            t = t.view(dtype)
        return t.to(dev)

    x = up(inp.x.view(np.int16), torch.bfloat16)
    logits = up(inp.logits)
    bias = up(inp.bias) if inp.bias is not None else None
    w13, s13 = up(inp.w13), up(inp.w13_scale.reshape(-1))
    w2, s2 = up(inp.w2), up(inp.w2_scale.reshape(-1))
    e13 = up(inp.w13_e8m0) if cfg.w_fp4 else None
    e2 = up(inp.w2_e8m0) if cfg.w_fp4 else None
    buf = moe.LayerBuffers.allocate(cfg.T, cfg.H, cfg.I, cfg.topk, cfg.num_local, cfg.act_quant,
                                    n_shared=cfg.n_shared)

    stages = STAGES

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record()
        mark(0)
        if cfg.n_shared:
            moe.moe_select_experts_shared(logits, bias, buf.topk_ids, buf.topk_weights,
                                          topk=cfg.topk, n_shared=cfg.n_shared,
                                          shared_weight=cfg.shared_weight, n_group=cfg.n_group,
                                          topk_group=cfg.topk_group, score_fn=cfg.score_fn,
                                          renormalize=cfg.renormalize,
                                          routed_scaling_factor=cfg.rsf, apply_rsf=cfg.apply_rsf)
        else:
            moe.moe_select_experts(logits, bias, buf.topk_ids, buf.topk_weights, topk=cfg.topk,
                                   n_group=cfg.n_group, topk_group=cfg.topk_group,
                                   score_fn=cfg.score_fn, renormalize=cfg.renormalize,
                                   routed_scaling_factor=cfg.rsf, apply_rsf=cfg.apply_rsf)
        mark(1)
        if cfg.n_shared:
            moe.moe_pre_reorder_quant_shared(x, buf.topk_ids, buf.a13, buf.a13_scale, buf.src2dst,
                                             buf.dst2src, buf.seg_indptr, buf.workspace,
                                             expert_start=cfg.expert_start, num_routed=cfg.num_local,
                                             shared_base=cfg.E, n_shared=cfg.n_shared,
                                             act_quant=cfg.act_quant)
        else:
            moe.moe_pre_reorder_quant(x, buf.topk_ids, buf.a13, buf.a13_scale, buf.src2dst,
                                      buf.dst2src, buf.seg_indptr, buf.workspace,
                                      expert_start=cfg.expert_start, num_local=cfg.num_local,
                                      act_quant=cfg.act_quant)
        mark(2)
        if cfg.w_fp4:
            moe.moe_grouped_gemm_mxfp4(buf.a13, buf.a13_scale, w13, e13, s13, buf.seg_indptr, buf.c13,
                                       act_quant=cfg.act_quant, w_quant=cfg.w_quant)
        else:
            moe.moe_grouped_gemm_fp8(buf.a13, buf.a13_scale, w13, s13, buf.seg_indptr, buf.c13,
                                     act_quant=cfg.act_quant, w_quant=cfg.w_quant)
        mark(3)
        moe.moe_act_requant(buf.c13, buf.seg_indptr, buf.a2, buf.a2_scale, buf.workspace,
                            act_quant=cfg.act_quant)
        mark(4)
        if cfg.w_fp4:
            moe.moe_grouped_gemm_mxfp4(buf.a2, buf.a2_scale, w2, e2, s2, buf.seg_indptr, buf.c2,
                                       act_quant=cfg.act_quant, w_quant=cfg.w_quant)
        else:
            moe.moe_grouped_gemm_fp8(buf.a2, buf.a2_scale, w2, s2, buf.seg_indptr, buf.c2,
                                     act_quant=cfg.act_quant, w_quant=cfg.w_quant)
        mark(5)
        moe.moe_post_reorder(buf.c2, buf.src2dst, buf.topk_weights, buf.out)
        mark(6)

    if graph:
        g = moe.LayerGraph(step, warmup=max(warmup, 1))
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t_start) * 1e3 / steps, None, buf, s13, s2

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` layer passes; HIP events on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(steps):
        step(ev[s])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / steps
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                for i, name in enumerate(stages)}

    return ms_per_step, stage_ms, buf, s13, s2


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs the layer on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import fp8_grouped_gemm_select_amd as moe
    import workloads as W

    cfg = W.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = W.gen_layer_inputs(cfg, seed=args.seed)

    gen_s = time.time() - t0
    print(f"[bench] {cfg.name}: inputs ready in {gen_s:.1f}s", file=sys.stderr, flush=True)
    # per-stage times: eager passes with HIP events between the stages
    eager_ms, stage_ms, buf, s13, s2 = time_layer(cfg, inp, args.steps, args.warmup, moe, torch, dev)
    # the headline: the same pass captured once in a HIP graph, `steps` replays timed
    # (the kernels and their arguments are those of the eager pass)
    if args.no_graph:
        ms_per_step = eager_ms
    else:
        ms_per_step, _, gbuf, _, _ = time_layer(cfg, inp, args.steps, args.warmup, moe, torch, dev,
                                                graph=True)
        del gbuf
    stages = STAGES
    seg = buf.seg_indptr.cpu().numpy()
    tokens_local = int((buf.src2dst.view(cfg.T, -1) >= 0).any(dim=1).sum())
    work, M, nonempty = algorithmic_work(cfg, seg, buf.a13_scale.numel() * 4, buf.a2_scale.numel() * 4,
                                         s13.numel(), s2.numel(), tokens_local)
    stage_stats = {}
    for name in stages:
        t = stage_ms[name] * 1e-3
        b, f = work[name]["bytes"], work[name]["flops"]
        stage_stats[name] = dict(us=round(stage_ms[name] * 1e3, 2), GBps=round(b / t / 1e9, 1),
                                 hbm_frac=round(b / t / 1e9 / HBM_PEAK_GBS, 4))
        if f:
            stage_stats[name].update(TFLOPs=round(f / t / 1e12, 1),
                                     mfma_frac=round(f / t / 1e12 / FP8_PEAK_TFLOPS, 4))
        # the stage's floor (bytes at HBM peak or FLOPs at MFMA peak, whichever is
        # longer) over its time: for a GEMM, its rate as a fraction of
        # min(MFMA peak, arithmetic intensity x HBM peak)
        stage_stats[name]["of_roofline"] = round(max(b / (HBM_PEAK_GBS * 1e9),
                                                     f / (FP8_PEAK_TFLOPS * 1e12)) / t, 4)
    dom = max(stages, key=lambda n: stage_ms[n])
    db, df = work[dom]["bytes"], work[dom]["flops"]
    dt = stage_ms[dom] * 1e-3
    hbm_time = db / (HBM_PEAK_GBS * 1e9)
    mfma_time = df / (FP8_PEAK_TFLOPS * 1e12) if df else 0.0
    if mfma_time > hbm_time:
        roof = dict(bound="mfma", achieved=round(df / dt / 1e12, 2), peak=FP8_PEAK_TFLOPS,
                    unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=round(db / dt / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = int(db)
    roof["algorithmic_flops"] = int(df)
    roof["traffic"] = measured_traffic(cfg.name, dom)
    gemm_t = (stage_ms["gemm_w13"] + stage_ms["gemm_w2"]) * 1e-3
    gemm_f = work["gemm_w13"]["flops"] + work["gemm_w2"]["flops"]
    gemm_floor = sum(max(work[n]["bytes"] / (HBM_PEAK_GBS * 1e9), work[n]["flops"] / (FP8_PEAK_TFLOPS * 1e12))
                     for n in ("gemm_w13", "gemm_w2"))
    gemm = dict(tflops=round(gemm_f / gemm_t / 1e12, 1),
                frac_of_fp8_peak=round(gemm_f / gemm_t / 1e12 / FP8_PEAK_TFLOPS, 4),
                frac_of_roofline=round(gemm_floor / gemm_t, 4),
                w13_tflops=stage_stats["gemm_w13"].get("TFLOPs"),
                w2_tflops=stage_stats["gemm_w2"].get("TFLOPs"))

    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1" if cfg.w_fp4 else "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "topk": cfg.topk, "num_local": cfg.num_local, "n_shared": cfg.n_shared, "M": M,
                   "experts_with_rows": nonempty, "act_quant": cfg.act_quant,
                   "w_quant": cfg.w_quant, "w_format": "mxfp4" if cfg.w_fp4 else "e4m3",
                   "parallelism": "single GPU (one EP share)"},
        "roofline": roof, "gemm": gemm, "stages": stage_stats,
        "launch": "eager" if args.no_graph else "hip_graph_replay",
        "eager": {"ms_per_step": round(eager_ms, 4), "tokens_per_s": round(cfg.T / (eager_ms * 1e-3), 1),
                  "note": "the same pass launched call by call with HIP events between stages "
                          "(source of the per-stage times)"},
    }

    if not args.no_next_rows:
        result["next_rows"] = {"router_select": time_router_select(cfg, inp, args, moe, W, torch, dev)}
        if cfg.name == "dsv3_prefill_ep":  # context: the same layer's decode share
            result["other_workloads"] = {"dsv3_decode_ep": time_other_layer(
                W.CONFIGS["dsv3_decode_ep"], args, moe, W, torch, dev,
                "the same layer at the decode share (T=128), timed on its own; not in value", graph=True)}
        fp4_name = cfg.name + "_fp4"
        if not cfg.w_fp4 and fp4_name in W.CONFIGS:
            del buf
            torch.cuda.empty_cache()
            result["next_rows"]["fp4_layer"] = time_fp4_layer(W.CONFIGS[fp4_name], args, moe, W, torch, dev)

    if not args.no_ceilings:
        ceil = measure_ceilings(torch, dev)
        result["ceilings"] = ceil
        meas = ceil["hbm_read_GBps"] if roof["bound"] == "hbm" else ceil["fp8_mfma_TFLOPs"]
        roof["measured_peak"] = meas
        roof["frac_of_measured"] = round(roof["achieved"] / meas, 4)
        gemm["frac_of_measured_mfma"] = round(gemm["tflops"] / ceil["fp8_mfma_TFLOPs"], 4)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


def time_fp4_layer(cfg, args, moe, W, torch, dev):
    """The same layer with MXFP4 expert weights, timed on its own (not in `value`)."""
    return time_other_layer(cfg, args, moe, W, torch, dev,
                            "MXFP4 expert weights (E2M1 + E8M0 per 32), same routing and activations; not in value")


def time_other_layer(cfg, args, moe, W, torch, dev, note, graph=False):
    """Another workload's whole layer, timed on its own (not in `value`); with
    graph=True also replayed from a HIP graph."""
    inp = W.gen_layer_inputs(cfg, seed=args.seed)
    ms_graph = None
    if graph:
        ms_graph, _, gbuf, _, _ = time_layer(cfg, inp, args.steps, args.warmup, moe, torch, dev, graph=True)
        del gbuf
    ms, stage_ms, buf, s13, s2 = time_layer(cfg, inp, args.steps, args.warmup, moe, torch, dev)
    seg = buf.seg_indptr.cpu().numpy()
    work, M, _ = algorithmic_work(cfg, seg, buf.a13_scale.numel() * 4, buf.a2_scale.numel() * 4,
                                  s13.numel(), s2.numel())
    out = dict(workload=cfg.name, tokens_per_s=round(cfg.T / (ms * 1e-3), 1), ms_per_step=round(ms, 4),
               M=int(M), note=note)
    if ms_graph is not None:  # the same pass replayed from a HIP graph (no per-launch host cost)
        out["graph"] = dict(tokens_per_s=round(cfg.T / (ms_graph * 1e-3), 1), ms_per_step=round(ms_graph, 4))
    for name in ("gemm_w13", "gemm_w2"):
        t = stage_ms[name] * 1e-3
        out[name] = dict(us=round(stage_ms[name] * 1e3, 2),
                         GBps=round(work[name]["bytes"] / t / 1e9, 1),
                         hbm_frac=round(work[name]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
                         TFLOPs=round(work[name]["flops"] / t / 1e12, 1),
                         mfma_frac=round(work[name]["flops"] / t / 1e12 / FP8_PEAK_TFLOPS, 4),
                         algorithmic_bytes=int(work[name]["bytes"]))
    del buf
    torch.cuda.empty_cache()
    return out


def time_router_select(cfg, inp, args, moe, W, torch, dev):
    """The router projection + stage 1 from the hidden states (an extension row,
    not part of the five-stage step): its own timed loop on the same stream."""
    wg = torch.from_numpy(W.gen_router_bf16(cfg, args.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    bias = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)
    ids = torch.empty(cfg.T, cfg.topk, dtype=torch.int32, device=dev)
    w = torch.empty(cfg.T, cfg.topk, dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.moe_router_workspace_bytes(cfg.T, cfg.H, cfg.E), 256), dtype=torch.uint8,
                     device=dev)

    def run():
        moe.moe_router_select(x, wg, bias, logits, ids, w, topk=cfg.topk, n_group=cfg.n_group,
                              topk_group=cfg.topk_group, score_fn=cfg.score_fn,
                              renormalize=cfg.renormalize, routed_scaling_factor=cfg.rsf,
                              apply_rsf=cfg.apply_rsf, workspace=ws)
    for _ in range(3):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / args.steps
    byts = cfg.T * cfg.H * 2 + cfg.E * cfg.H * 2 + 2 * cfg.T * cfg.E * 4 + cfg.T * cfg.topk * 8
    flops = 2 * cfg.T * cfg.H * cfg.E
    return dict(us=round(t * 1e6, 2), GBps=round(byts / t / 1e9, 1), hbm_frac=round(byts / t / 1e9 / HBM_PEAK_GBS, 4),
                TFLOPs=round(flops / t / 1e12, 1), bf16_mfma_frac=round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                algorithmic_bytes=int(byts), flops=int(flops),
                note="bf16 router projection x @ wg^T + stage 1, timed on its own, not in value")


def measure_ceilings(torch, dev, nbytes=2 << 30, mfma_iters=2000, reps=5):
    """What this GPU reaches with plain kernels (libmoe_ceilings.so): a streaming
    copy and a streaming read of `nbytes` (HBM GB/s; the copy counts its bytes
    read and written; the read is timed with ordinary and with nontemporal loads
    and the faster one is the ceiling) and a loop of independent 16x16x128 FP8 MFMAs on every CU
    at two waves per SIMD (TFLOP/s, and the shader clock it held). Each is the
    mean of `reps` timed launches after two untimed ones."""
    import ctypes
    from fp8_grouped_gemm_select_amd import _build
    lib = ctypes.CDLL(_build.CEIL_LIB)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.ceil_stream_copy.argtypes = [P, P, I64, P]
    lib.ceil_stream_read.argtypes = [P, I64, P, P]
    lib.ceil_stream_read_nt.argtypes = [P, I64, P, P]
    lib.ceil_mfma_loop.argtypes = [I32, P, P, P]
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    small = torch.zeros(64, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def timed(launch):
        for _ in range(2):
            launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            launch()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def check(rc):
        if rc < 0:
            raise RuntimeError(f"ceiling kernel launch failed ({rc})")
        return rc

    t_copy = timed(lambda: check(lib.ceil_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream)))
    t_read = timed(lambda: check(lib.ceil_stream_read(src.data_ptr(), nbytes, small.data_ptr(), stream)))
    t_read_nt = timed(lambda: check(lib.ceil_stream_read_nt(src.data_ptr(), nbytes, small.data_ptr(), stream)))
    blocks = [0]
    t_mfma = timed(lambda: blocks.__setitem__(0, check(lib.ceil_mfma_loop(
        mfma_iters, small.data_ptr(), small[8:].data_ptr(), stream))))
    clk = small[8:10].cpu().numpy()
    flops = float(blocks[0]) * 8 * mfma_iters * 16 * 65536
    del src, dst
    torch.cuda.empty_cache()
    return dict(hbm_copy_GBps=round(2 * nbytes / t_copy / 1e9, 1),
                hbm_read_GBps=round(nbytes / min(t_read, t_read_nt) / 1e9, 1),
                hbm_read_plain_GBps=round(nbytes / t_read / 1e9, 1),
                hbm_read_nontemporal_GBps=round(nbytes / t_read_nt / 1e9, 1),
                fp8_mfma_TFLOPs=round(flops / t_mfma / 1e12, 1),
                mfma_clock_GHz=round(float(clk[0]) / (float(clk[1]) / 100e6) / 1e9, 3),
                note=f"plain kernels on this GPU: copy and read of {nbytes >> 20} MiB (hbm_read_GBps: the "
                     f"faster of ordinary and nontemporal loads), 16x16x128 FP8 MFMA loop (two waves per "
                     f"SIMD); not in value")


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when there is none or the
    stage's kernel source has changed since the counters were taken."""
    from fp8_grouped_gemm_select_amd import profsum
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    st = t.get("stages", {}).get(stage)
    if not st or st.get("source_sha256") != profsum.source_hash(stage):
        return None
    return st["traffic_bytes"]


def cpu_baseline(cfg, inp, sample_tokens):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the same workload."""
    import dataclasses
    import oracle
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    if not sample_tokens:
        sample_tokens = {"tiny": 16, "dsv3_decode_ep": 128, "dsv3_prefill_ep": 4096,
                         "mixtral": 64, "skewed_block": 512}.get(cfg.name, 256)
    Ts = min(sample_tokens, cfg.T)
    sub = dataclasses.replace(inp, cfg=dataclasses.replace(cfg, T=Ts), x=inp.x[:Ts],
                              logits=inp.logits[:Ts])
    t0 = time.perf_counter()
    oracle.layer(sub)
    dt = time.perf_counter() - t0
    return {"value": round(Ts / dt, 2), "unit": "tokens/s", "cores": oracle.get_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {Ts} of {cfg.T} tokens of {cfg.name}, full expert weights, "
                      f"whole layer (routing, permutation, both GEMMs, activation, combine)"}


if __name__ == "__main__":
    main()
