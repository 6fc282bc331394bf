"""Pins for the oracle's forward: dense brute force, a textbook dense FFN,
closed forms and special cases."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth


def _inputs(T, d, E, k, h, seed=3, ls=1.0, xs=1.0, ws=0.1):
    return dict(logits=synth.normal((T, E), seed, 0, ls), x=synth.normal((T, d), seed, 1, xs),
                w1=synth.normal((E, 2 * h, d), seed, 2, ws), w2=synth.normal((E, d, h), seed, 3, ws),
                dout=synth.normal((T, d), seed, 4, 1.0))


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("shape", [(64, 32, 4, 2, 48), (40, 16, 6, 6, 16), (30, 32, 8, 1, 32)])
def test_dense_brute_force(dtype, shape):
    T, d, E, k, h = shape
    inp = _inputs(T, d, E, k, h)
    f = oracle.layer_forward(inp, k, dtype)
    b = brute.dense_forward(inp["logits"], inp["x"], inp["w1"], inp["w2"], k, dtype)
    # y rows: the oracle's y_perm row p equals expert e's output on token sorted_token[p]
    e_of = oracle.expert_of_rows(f["route"]["counts"])
    y_b = b["y_all"][e_of, f["route"]["sorted_token"]]
    if dtype == "bf16":
        # fp64 sums in different orders can straddle a bf16 rounding boundary:
        # allow isolated one-ulp differences, nothing more
        ulp = np.abs(brute.round_bf16(y_b * (1 + 2 ** -8)) - y_b) + 1e-30
        assert np.all(np.abs(f["y_perm"] - y_b) <= ulp)
        assert (f["y_perm"] != y_b).mean() < 1e-3
        assert _rel(f["out"], b["out"]) < 1e-2
    else:
        assert _rel(f["y_perm"], y_b) < 1e-12 if dtype == "f64" else _rel(f["y_perm"], y_b) < 1e-6
        assert _rel(f["out"], b["out"]) < (1e-12 if dtype == "f64" else 1e-6)


def test_cfg1_tiny_fp32_against_brute_force():
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.host_inputs(w, 0)
    f = oracle.layer_forward(inp, w.k, "f32")
    b = brute.dense_forward(inp["logits"], inp["x"], inp["w1"], inp["w2"], w.k, "f32")
    assert _rel(f["out"], b["out"]) < 1e-6
    c = f["route"]["counts"]
    assert c.sum() == w.R and c.min() > 0


def test_single_expert_is_dense_swiglu_ffn():
    """E=1, k=1: gate 1 and the layer is one dense SwiGLU FFN (torch, fp64)."""
    T, d, h = 24, 16, 20
    inp = _inputs(T, d, 1, 1, h)
    f = oracle.layer_forward(inp, 1, "f64")
    X = torch.tensor(inp["x"], dtype=torch.float64)
    W1 = torch.tensor(inp["w1"][0], dtype=torch.float64)
    W2 = torch.tensor(inp["w2"][0], dtype=torch.float64)
    pre = torch.matmul(X, W1.T)
    ref = torch.matmul(torch.nn.functional.silu(pre[:, :h]) * pre[:, h:], W2.T).numpy()
    assert np.all(f["route"]["topk_gate"] == 1.0)
    assert _rel(f["out"], ref) < 1e-12


def test_closed_form_one_by_one():
    """d = h = 1: out = g0*silu(x wg0)(x wu0) w2_0 + g1*silu(x wg1)(x wu1) w2_1."""
    x = np.array([[1.5]], np.float32)
    logits = np.array([[0.25, -0.25]], np.float32)
    w1 = np.array([[[0.5], [2.0]], [[-1.0], [0.25]]], np.float32)
    w2 = np.array([[[3.0]], [[-2.0]]], np.float32)
    f = oracle.layer_forward(dict(logits=logits, x=x, w1=w1, w2=w2), 2, "f64")
    silu = lambda a: a / (1 + np.exp(-a))
    g0 = 1 / (1 + np.exp(-0.5))          # softmax of (0.25, -0.25)
    y0 = silu(1.5 * 0.5) * (1.5 * 2.0) * 3.0
    y1 = silu(1.5 * -1.0) * (1.5 * 0.25) * -2.0
    ref = np.float32(g0) * y0 + np.float32(1 - g0) * y1
    assert abs(f["out"][0, 0] - ref) < 1e-7


def test_k_equals_E_every_token_uses_every_expert():
    T, d, E, h = 20, 16, 4, 8
    inp = _inputs(T, d, E, E, h)
    f = oracle.layer_forward(inp, E, "f64")
    assert np.all(f["route"]["counts"] == T)
    # dense mixture with the full softmax as weights
    l = inp["logits"].astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    b = brute.dense_forward(inp["logits"], inp["x"], inp["w1"], inp["w2"], E, "f64")
    assert _rel(f["out"], b["out"]) < 1e-12
    assert np.allclose(np.sort(f["route"]["topk_gate"], 1), np.sort(p, 1), atol=1e-7)


def test_permute_is_row_gather_and_identity_back():
    T, d, E, k, h = 50, 8, 5, 2, 8
    inp = _inputs(T, d, E, k, h)
    f = oracle.layer_forward(inp, k, "f32")
    r = f["route"]
    # x_perm[token_pos[t,j]] == X[t]
    for j in range(k):
        assert np.array_equal(f["x_perm"][r["token_pos"][:, j]], inp["x"].astype(np.float64))


def test_empty_experts_and_zero_tokens():
    T, d, E, k, h = 16, 8, 6, 1, 8
    inp = _inputs(T, d, E, k, h)
    inp["logits"][:, 2] += 50.0
    f = oracle.layer_forward(inp, k, "f32")
    assert f["route"]["counts"][2] == T
    b = brute.dense_forward(inp["logits"], inp["x"], inp["w1"], inp["w2"], k, "f32")
    assert _rel(f["out"], b["out"]) < 1e-6
    z = _inputs(0, d, E, k, h)
    f0 = oracle.layer_forward(z, k, "f32")
    assert f0["out"].shape == (0, d)


def test_capacity_padding_baseline():
    """Padded-capacity alternative (kongchang.com, 'routing is a systems problem'):
    a capacity no expert exceeds changes nothing; capacity 0 drops everything;
    otherwise exactly the rows ranked >= C inside their expert vanish."""
    T, d, E, k, h = 60, 8, 4, 2, 8
    inp = _inputs(T, d, E, k, h)
    full = oracle.layer_forward(inp, k, "f64")
    big = oracle.layer_forward(inp, k, "f64", capacity=T)
    assert np.array_equal(full["out"], big["out"])
    zero = oracle.layer_forward(inp, k, "f64", capacity=0)
    assert np.all(zero["out"] == 0)
    C = 20
    cap = oracle.layer_forward(inp, k, "f64", capacity=C)
    r = full["route"]
    ref = np.zeros_like(full["out"])
    for t in range(T):
        for j in range(k):
            e = r["topk_idx"][t, j]
            rank = r["token_pos"][t, j] - r["offsets"][e]
            if rank < C:
                ref[t] += r["topk_gate"][t, j] * full["y_perm"][r["token_pos"][t, j]]
    assert _rel(cap["out"], ref) < 1e-12
