"""Pins for the oracle's backward: torch autograd on the dense layer (fp64,
CPU), central finite differences, and the sampled form against the full one."""
import numpy as np
import pytest

import oracle
from oracle import brute
import synth


def _inputs(T, d, E, k, h, seed=5, ls=1.0, ws=0.2):
    return dict(logits=synth.normal((T, E), seed, 0, ls), x=synth.normal((T, d), seed, 1, 1.0),
                w1=synth.normal((E, 2 * h, d), seed, 2, ws), w2=synth.normal((E, d, h), seed, 3, ws),
                dout=synth.normal((T, d), seed, 4, 1.0))


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("shape", [(48, 16, 4, 2, 24), (30, 8, 8, 3, 16), (20, 16, 3, 3, 8)])
def test_against_autograd(shape):
    T, d, E, k, h = shape
    inp = _inputs(T, d, E, k, h)
    f = oracle.layer_forward(inp, k, "f64")
    b = oracle.layer_backward(inp, f, k, "f64")
    ref = brute.autograd_layer(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dout"], k)
    # gates are stored in fp32 (a rounding point of the layer); all else is fp64
    assert _rel(f["out"], ref["out"]) < 1e-6
    assert _rel(b["dx"], ref["dx"]) < 1e-6
    # dW and dlogits are stored in fp32
    assert _rel(b["dW1"], ref["dW1"]) < 1e-6
    assert _rel(b["dW2"], ref["dW2"]) < 1e-6
    assert _rel(b["dlogits"], ref["dlogits"]) < 1e-6
    # unselected experts get exactly zero logit gradient
    r = f["route"]
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, r["topk_idx"].astype(np.int64), True, 1)
    assert np.all(b["dlogits"][~sel] == 0)


def test_empty_expert_gets_zero_weight_gradient():
    T, d, E, k, h = 24, 8, 5, 1, 8
    inp = _inputs(T, d, E, k, h)
    inp["logits"][:, 4] -= 100.0      # nobody picks expert 4
    f = oracle.layer_forward(inp, k, "f32")
    b = oracle.layer_backward(inp, f, k, "f32")
    assert f["route"]["counts"][4] == 0
    assert np.all(b["dW1"][4] == 0) and np.all(b["dW2"][4] == 0)


def test_finite_differences():
    """Central differences of L = <dOut, out> along random directions (fp64,
    no storage rounding); logit directions only touch tokens whose k-th/k+1-th
    margin is large, so the selection cannot flip."""
    T, d, E, k, h = 16, 8, 4, 2, 8
    inp = _inputs(T, d, E, k, h)
    f = oracle.layer_forward(inp, k, "f64")
    b = oracle.layer_backward(inp, f, k, "f64")
    rng = np.random.default_rng(11)
    eps = 1e-6

    def loss(mod):
        x = dict(inp)
        x.update(mod)
        return float((oracle.layer_forward(x, k, "f64")["out"] * inp["dout"]).sum())

    srt = -np.sort(-inp["logits"].astype(np.float64), 1)
    safe = (srt[:, k - 1] - srt[:, k]) > 1e-2
    grads = dict(x=b["dx"], w1=b["dW1"], w2=b["dW2"], logits=b["dlogits"])
    for name in ("x", "w1", "w2", "logits"):
        for _ in range(4):
            v = rng.standard_normal(inp[name].shape)
            if name == "logits":
                v[~safe] = 0.0
            base = inp[name].astype(np.float64)
            # gates are stored in fp32, so logit steps must dwarf their rounding
            h_, tol = (1e-3, 1e-3) if name == "logits" else (eps, 1e-5)
            lp = loss({name: base + h_ * v})
            lm = loss({name: base - h_ * v})
            fd = (lp - lm) / (2 * h_)
            an = float((grads[name] * v).sum())
            assert abs(fd - an) <= tol * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sampled_equals_full(dtype):
    """layer_sampled reproduces the full layer's values for chosen tokens/experts."""
    T, d, E, k, h = 64, 16, 8, 2, 16
    inp = _inputs(T, d, E, k, h)
    f = oracle.layer_forward(inp, k, dtype)
    b = oracle.layer_backward(inp, f, k, dtype)
    toks = np.array([0, 5, 17, 63])
    exps = np.array([1, 6])
    s = oracle.layer_sampled(inp, k, dtype, toks, exps)
    assert np.array_equal(s["out"], f["out"][toks])
    assert np.array_equal(s["dx"], b["dx"][toks])
    assert np.array_equal(s["dlogits"], b["dlogits"][toks])
    for e in exps:
        assert np.array_equal(s["dW1"][e], b["dW1"][e])
        assert np.array_equal(s["dW2"][e], b["dW2"][e])


def test_capacity_backward_matches_autograd_of_dropped_layer():
    """With a capacity, dropped rows carry no gradient (pin by autograd on the
    dense form with those (token, expert) pairs masked out)."""
    import torch
    T, d, E, k, h = 40, 8, 4, 2, 8
    inp = _inputs(T, d, E, k, h)
    C = 12
    f = oracle.layer_forward(inp, k, "f64", capacity=C)
    b = oracle.layer_backward(inp, f, k, "f64")
    r = f["route"]
    keep = f["keep"]
    L = torch.tensor(inp["logits"].astype(np.float64), requires_grad=True)
    X = torch.tensor(inp["x"].astype(np.float64), requires_grad=True)
    W1 = torch.tensor(inp["w1"].astype(np.float64), requires_grad=True)
    W2 = torch.tensor(inp["w2"].astype(np.float64), requires_grad=True)
    idx = torch.from_numpy(r["topk_idx"].astype(np.int64))
    g = torch.softmax(torch.gather(L, 1, idx), 1) * torch.from_numpy(keep.astype(np.float64))
    mask = torch.zeros(T, E, dtype=torch.float64).scatter(1, idx, g)
    out = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        pre = X @ W1[e].T
        out = out + mask[:, e:e + 1] * ((torch.nn.functional.silu(pre[:, :h]) * pre[:, h:]) @ W2[e].T)
    (out * torch.tensor(inp["dout"].astype(np.float64))).sum().backward()
    assert _rel(f["out"], out.detach().numpy()) < 1e-6
    assert _rel(b["dx"], X.grad.numpy()) < 1e-6
    assert _rel(b["dW1"], W1.grad.numpy()) < 1e-6
    assert _rel(b["dlogits"], L.grad.numpy()) < 1e-6
