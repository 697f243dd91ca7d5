"""Pins for the oracle's fused gate (select_experts) and permutation.

Brute force over every subset on tiny inputs, hand-worked golden cases, ties,
and the special cases that reduce to plain top-k / softmax.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _sig64(x):
    return 1.0 / (1.0 + math.exp(-x))


def _load_golden():
    cases, cur = [], None
    for line in open(os.path.join(HERE, "golden", "routing_hand.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
        elif key in ("logits", "bias"):
            cur[key] = np.array([float(v) for v in vals], dtype=np.float32)
        elif key == "ids":
            cur[key] = [int(v) for v in vals]
        else:
            cur[key] = int(vals[0])
    return cases


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_grouped_topk_hand_cases(case):
    ids, w = oracle.select_experts(case["logits"][None, :], case["bias"], case["topk"],
                                   case["n_group"], case["topk_group"], W.SCORE_SIGMOID, 1, 1.0, 1)
    assert list(ids[0]) == case["ids"]
    s = np.array([_sig64(case["logits"][i]) for i in case["ids"]])
    np.testing.assert_allclose(w[0], s / s.sum(), rtol=1e-6)


def test_softmax_topk_brute_force_all_pairs():
    """E=8, k=2: the chosen pair is the one of the 28 with the two largest logits."""
    g = np.random.default_rng(0)
    logits = g.standard_normal((300, 8)).astype(np.float32)
    ids, w = oracle.select_experts(logits, None, 2, score_fn=W.SCORE_SOFTMAX)
    for t in range(logits.shape[0]):
        best = max(itertools.combinations(range(8), 2),
                   key=lambda p: (sorted(logits[t, list(p)])[0], sorted(logits[t, list(p)])[1]))
        assert set(ids[t]) == set(best)
        assert logits[t, ids[t, 0]] >= logits[t, ids[t, 1]]
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-6)


def test_grouped_topk_brute_force_subsets():
    """E=16, 4 groups, keep 2, k=4, with bias: exhaustive over group pairs and expert subsets."""
    g = np.random.default_rng(1)
    E, NG, TG, K = 16, 4, 2, 4
    logits = g.standard_normal((200, E)).astype(np.float32)
    bias = (g.standard_normal(E) * 0.3).astype(np.float32)
    ids, w = oracle.select_experts(logits, bias, K, NG, TG, W.SCORE_SIGMOID, 1, 2.5, 1)
    for t in range(logits.shape[0]):
        s = np.array([oracle.sigmoid(float(v)) for v in logits[t]], dtype=np.float32)
        c = (s + bias).astype(np.float32)
        gscore = [float(np.float32(sum(sorted(c[4 * q:4 * q + 4])[-2:]))) for q in range(NG)]
        best_groups = max(itertools.combinations(range(NG), TG),
                          key=lambda gg: sorted([gscore[q] for q in gg], reverse=True))
        cand = [e for q in best_groups for e in range(4 * q, 4 * q + 4)]
        best_set = max(itertools.combinations(cand, K), key=lambda ss: sum(c[list(ss)].astype(np.float64)))
        assert set(ids[t]) == set(best_set), t
        ordered = sorted(ids[t], key=lambda e: (-c[e], e))
        assert list(ids[t]) == ordered
        sv = s[ids[t]].astype(np.float64)
        np.testing.assert_allclose(w[t], 2.5 * sv / sv.sum(), rtol=1e-6)


def test_ties_go_to_lower_id():
    logits = np.array([[1, 3, 3, 0, 3, 0, 0, 1]], dtype=np.float32)
    ids, _ = oracle.select_experts(logits, None, 4, score_fn=W.SCORE_SOFTMAX)
    assert list(ids[0]) == [1, 2, 4, 0]
    ids, _ = oracle.select_experts(logits, np.zeros(8, np.float32), 4, 1, 1, W.SCORE_SIGMOID)
    assert list(ids[0]) == [1, 2, 4, 0]


def test_one_group_is_plain_topk():
    g = np.random.default_rng(2)
    logits = g.standard_normal((64, 32)).astype(np.float32)
    bias = (g.standard_normal(32) * 0.1).astype(np.float32)
    a, wa = oracle.select_experts(logits, bias, 6, 1, 1, W.SCORE_SIGMOID)
    b, wb = oracle.select_experts(logits, bias, 6, 4, 4, W.SCORE_SIGMOID)  # all groups kept
    assert np.array_equal(a, b) and np.array_equal(wa, wb)
    for t in range(64):
        s = np.array([oracle.sigmoid(float(v)) for v in logits[t]], dtype=np.float32)
        c = s + bias
        ref = sorted(range(32), key=lambda e: (-c[e], e))[:6]
        assert list(a[t]) == ref


def test_k_equals_e_gives_softmax():
    g = np.random.default_rng(3)
    logits = g.standard_normal((16, 8)).astype(np.float32)
    ids, w = oracle.select_experts(logits, None, 8, score_fn=W.SCORE_SOFTMAX)
    for t in range(16):
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=1e-6)
        assert sorted(ids[t]) == list(range(8))


def test_routed_scaling_factor_applied_exactly_once():
    g = np.random.default_rng(4)
    logits = g.standard_normal((256, 256)).astype(np.float32)
    bias = (g.standard_normal(256) * 0.01).astype(np.float32)
    i1, w1 = oracle.select_experts(logits, bias, 8, 8, 4, W.SCORE_SIGMOID, 1, 1.0, 1)
    i2, w2 = oracle.select_experts(logits, bias, 8, 8, 4, W.SCORE_SIGMOID, 1, 2.5, 1)
    i0, w0 = oracle.select_experts(logits, bias, 8, 8, 4, W.SCORE_SIGMOID, 1, 2.5, 0)
    assert np.array_equal(i1, i2) and np.array_equal(i1, i0)
    np.testing.assert_array_equal(w0, w1)
    np.testing.assert_allclose(w2, 2.5 * w1.astype(np.float64), rtol=2 ** -23)
    np.testing.assert_allclose(w2.astype(np.float64).sum(1), 2.5, rtol=4 * 2 ** -23)
    np.testing.assert_allclose(w1.astype(np.float64).sum(1), 1.0, rtol=4 * 2 ** -23)


def test_unnormalised_weights():
    g = np.random.default_rng(9)
    logits = g.standard_normal((8, 16)).astype(np.float32)
    ids, w = oracle.select_experts(logits, None, 3, 1, 1, W.SCORE_SIGMOID, 0, 1.0, 0)
    for t in range(8):
        ref = [oracle.sigmoid(float(logits[t, e])) for e in ids[t]]
        np.testing.assert_array_equal(w[t], np.array(ref, np.float32))
    ids, w = oracle.select_experts(logits, None, 3, score_fn=W.SCORE_SOFTMAX, renormalize=0)
    for t in range(8):
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(w[t], p[ids[t]], rtol=1e-6)


def test_invalid_routing_arguments_rejected():
    logits = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.select_experts(logits, None, 9)
    with pytest.raises(ValueError):
        oracle.select_experts(logits, None, 2, 3, 1, W.SCORE_SIGMOID)  # 8 % 3 != 0
    with pytest.raises(ValueError):
        oracle.select_experts(logits, None, 4, 4, 1, W.SCORE_SIGMOID)  # 1 group of 2 < 4


# ---- permutation ------------------------------------------------------------

@pytest.mark.parametrize("expert_start,num_local", [(0, 16), (0, 4), (5, 6), (12, 4), (0, 1)])
def test_permutation_invariants(expert_start, num_local):
    g = np.random.default_rng(10 + expert_start)
    T, E, K = 97, 16, 4
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    m_cap = T * min(K, num_local)
    src2dst, dst2src, seg = oracle.permute(ids, expert_start, num_local, m_cap)
    flat = ids.reshape(-1)
    local = (flat >= expert_start) & (flat < expert_start + num_local)
    M = int(local.sum())
    counts = np.bincount(flat[local] - expert_start, minlength=num_local)
    assert np.array_equal(seg, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    assert seg[-1] == M
    assert np.all(src2dst[~local] == -1)
    f_local = np.nonzero(local)[0]
    assert np.array_equal(dst2src[src2dst[f_local]], f_local)
    assert np.array_equal(src2dst[dst2src[:M]], np.arange(M))
    assert np.all(dst2src[M:] == -1)
    for e in range(num_local):
        rows = dst2src[seg[e]:seg[e + 1]]
        assert np.all(np.diff(rows) > 0)
        assert np.all(flat[rows] == expert_start + e)


def test_permutation_empty_and_no_local():
    ids = np.zeros((0, 2), np.int32)
    s2d, d2s, seg = oracle.permute(ids, 0, 4, 0)
    assert s2d.size == 0 and np.all(seg == 0)
    ids = np.array([[5, 6], [7, 5]], np.int32)
    s2d, d2s, seg = oracle.permute(ids, 0, 4, 4)
    assert np.all(s2d == -1) and np.all(seg == 0) and np.all(d2s == -1)
