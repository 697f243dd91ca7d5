"""Host-side checks of bench.py: the one-GPU guard and the algorithmic byte and
flop counts the roofline is priced on (no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _seg(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def test_gemm_work_counts_weights_of_experts_with_rows_only():
    cfg = W.CONFIGS["dsv3_prefill_ep"]
    counts = np.zeros(cfg.num_local, np.int64)
    counts[:3] = [100, 50, 7]            # three experts with rows
    seg = _seg(counts)
    M = int(seg[-1])
    work, m, nonempty = bench.algorithmic_work(cfg, seg, M * 4, M * 4, cfg.num_local * 2 * cfg.I,
                                               cfg.num_local * cfg.H)
    assert (m, nonempty) == (M, 3)
    H, I = cfg.H, cfg.I
    w13 = 3 * 2 * I * H + 3 * 2 * I * 4                       # codes + per-channel scales
    assert work["gemm_w13"]["bytes"] == M * H + M * 4 + w13 + M * 2 * I * 2 + (cfg.num_local + 1) * 4
    assert work["gemm_w13"]["flops"] == 2 * M * 2 * I * H
    assert work["gemm_w2"]["flops"] == 2 * M * H * I


def test_fp4_weight_bytes_are_half_a_byte_plus_the_block_scales():
    cfg = W.CONFIGS["dsv3_prefill_ep_fp4"]
    seg = _seg(np.full(cfg.num_local, 10))
    work8, _, _ = bench.algorithmic_work(W.CONFIGS["dsv3_prefill_ep"], seg, 0, 0, 0, 0)
    work4, _, _ = bench.algorithmic_work(cfg, seg, 0, 0, 0, 0)
    w8 = cfg.num_local * 2 * cfg.I * cfg.H
    assert work8["gemm_w13"]["bytes"] - work4["gemm_w13"]["bytes"] == w8 - int(w8 * (0.5 + 1 / 32))
