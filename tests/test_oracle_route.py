"""Pins for the oracle's routing (top-k, gates, counts, offsets, positions).

The pages fix only that each token activates k of E experts (kongchang.com,
"capacity tax") and that split sizes and group sizes are routing metadata
(kongchang.com, "routing is a systems problem"). The rest is pinned by a hand-
derived example, by an independent brute force (full stable sort + per-expert
listing), exhaustive tie cases and invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _check_invariants(r, logits, k):
    T, E = logits.shape
    idx, gate, pos = r["topk_idx"], r["topk_gate"], r["token_pos"]
    R = T * k
    assert r["counts"].sum() == R
    assert r["offsets"][0] == 0 and r["offsets"][-1] == R
    assert np.all(np.diff(r["offsets"]) == r["counts"])
    for t in range(T):
        assert len(set(idx[t].tolist())) == k                       # k distinct experts
        sel = logits[t, idx[t]]
        assert np.all(sel[:-1] >= sel[1:])                          # non-increasing
        unsel = np.setdiff1d(np.arange(E), idx[t])
        if len(unsel):
            assert logits[t, unsel].max() <= sel[-1]                # nothing better left out
    assert abs(gate.astype(np.float64).sum(1) - 1).max() <= k * 2.0 ** -23
    assert np.all(gate > 0) or np.all(gate >= 0)
    # token_pos is a bijection onto [0, R) and sorted_* are its inverse
    flat = pos.reshape(-1)
    assert np.array_equal(np.sort(flat), np.arange(R))
    st, ss = r["sorted_token"], r["sorted_slot"]
    for t in range(T):
        for j in range(k):
            p = pos[t, j]
            assert st[p] == t and ss[p] == j
            e = idx[t, j]
            assert r["offsets"][e] <= p < r["offsets"][e + 1]
    # inside each group, tokens strictly increase
    for e in range(E):
        seg = st[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLD, "route_tiny.json")))
    logits = np.array([[float(v) for v in row] for row in g["logits"]], np.float32)
    assert np.signbit(logits[2, 0]) and not np.signbit(logits[2, 1])
    r = oracle.route(logits, g["k"], g["tile_m"])
    for key in ("topk_idx", "counts", "offsets", "tile_offsets", "token_pos", "sorted_token",
                "sorted_slot"):
        assert np.array_equal(r[key], np.array(g[key])), key
    assert np.allclose(r["topk_gate"], np.array(g["topk_gate"]), rtol=0, atol=1e-7)


@pytest.mark.parametrize("T,E,k,scale", [(256, 8, 2, 0.02), (300, 16, 3, 1.0), (97, 128, 4, 1.0),
                                         (64, 5, 5, 1.0), (33, 1, 1, 1.0), (0, 8, 2, 1.0)])
def test_matches_brute_force(T, E, k, scale):
    logits = synth.normal((T, E), 7, 0, scale)
    r = oracle.route(logits, k, 16)
    b = brute.route(logits, k, 16)
    for key in ("topk_idx", "counts", "offsets", "tile_offsets", "token_pos", "sorted_token",
                "sorted_slot"):
        assert np.array_equal(r[key], b[key]), key
    # gates: same value by two formulas (selected softmax vs renormalised full softmax)
    assert np.allclose(r["topk_gate"], b["topk_gate"], rtol=2e-7, atol=0)
    if T:
        _check_invariants(r, logits, k)


@pytest.mark.parametrize("vals", [(0.0, 1.0, 2.0), (-0.0, 0.0)])
def test_exhaustive_ties(vals):
    """Every logit row over `vals` for E=4 (and tiny T) matches the brute force."""
    E = 4
    rows = np.array(list(itertools.product(vals, repeat=E)), np.float32)
    for k in range(1, E + 1):
        r = oracle.route(rows, k, 3)
        b = brute.route(rows, k, 3)
        for key in ("topk_idx", "token_pos", "counts", "tile_offsets"):
            assert np.array_equal(r[key], b[key]), (k, key)
        _check_invariants(r, rows, k)


def test_all_equal_logits():
    """Identical logits everywhere: experts 0..k-1 get T rows each, the rest 0."""
    T, E, k = 50, 8, 3
    r = oracle.route(np.full((T, E), 0.25, np.float32), k)
    assert np.array_equal(r["counts"], [T] * k + [0] * (E - k))
    assert np.allclose(r["topk_gate"], 1.0 / k)


def test_one_hot_skew():
    """Every token prefers expert 5: it gets all T rows."""
    T, E = 40, 8
    logits = synth.normal((T, E), 1, 0, 0.1)
    logits[:, 5] += 100.0
    r = oracle.route(logits, 1)
    assert r["counts"][5] == T and r["counts"].sum() == T
    assert np.array_equal(r["sorted_token"], np.arange(T))


def test_zipf_workload_shape():
    """The skewed workload's generator yields empty experts and hot experts."""
    w = synth.WORKLOADS["e128_bf16_zipf"]
    logits = synth.normal((w.T, w.E), 0, synth.STREAM_LOGITS, 1.0) + synth.zipf_bias(w.E, 1.2)
    r = oracle.route(logits, w.k)
    mean = w.R / w.E
    assert (r["counts"] == 0).sum() > 10
    assert (r["counts"] > 10 * mean).sum() >= 2
