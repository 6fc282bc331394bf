"""Pins for the oracle's MXFP8 layer: an independent dense form that
quantises with torch's float8_e4m3fn cast, plus planted mistakes in the
oracle's wiring (a tensor quantised along the wrong axis, a quantisation
skipped) that the pin must catch."""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth


def _inp(T=80, d=128, E=4, k=2, h=64, seed=9):
    inp = dict(logits=synth.normal((T, E), seed, 0, 1.0), x=synth.normal((T, d), seed, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), seed, 2, 0.05),
               w2=synth.normal((E, d, h), seed, 3, 0.05), dout=synth.normal((T, d), seed, 4, 1.0))
    for key in ("x", "dout"):
        inp[key] = torch.from_numpy(inp[key]).bfloat16().float().numpy()
    return inp


def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


def _compare(m, ref, E, tol=1e-6):
    assert _rel(m["out"], ref["out"]) < tol
    assert _rel(m["dx"], ref["dx"]) < tol
    assert _rel(m["dlogits"], ref["dlogits"]) < tol
    for e in range(E):
        assert _rel(m["dW1"][e], ref["dW1"][e]) < tol, e
        assert _rel(m["dW2"][e], ref["dW2"][e]) < tol, e


def test_quantise_round_trip_matches_torch_cast():
    a = (np.random.default_rng(1).standard_normal((40, 96)) *
         np.exp(np.random.default_rng(2).uniform(-8, 8, (40, 1)))).astype(np.float32)
    assert np.array_equal(oracle.mx_rows(a), brute.mx_rows_torch(a))
    assert np.array_equal(oracle.mx_cols(a), brute.mx_cols_torch(a))


@pytest.mark.parametrize("shape", [(80, 128, 4, 2, 64), (50, 256, 6, 3, 128)])
def test_mx_layer_matches_dense_torch_form(shape):
    T, d, E, k, h = shape
    inp = _inp(T, d, E, k, h)
    m = oracle.layer_mx(inp, k)
    ref = brute.mx_layer(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dout"], k)
    # the same definitions in fp64 with a different summation order: rare
    # one-ulp bf16 flips of a stored intermediate are the only differences
    assert _rel(m["out"], ref["out"]) < 2e-2
    assert (np.abs(m["out"] - ref["out"]) > 1e-12).mean() < 5e-3
    for key in ("dx", "dlogits"):
        assert _rel(m[key], ref[key]) < 2e-2, key
        assert (np.abs(m[key] - ref[key]) > 1e-6 * np.abs(ref[key]).max()).mean() < 2e-2, key
    for e in range(E):
        assert _rel(m["dW1"][e], ref["dW1"][e]) < 2e-2
        assert _rel(m["dW2"][e], ref["dW2"][e]) < 2e-2


def test_sampled_equals_full():
    inp = _inp()
    full = oracle.layer_mx(inp, 2)
    toks, exps = np.array([0, 7, 79]), np.array([1, 3])
    s = oracle.layer_mx(inp, 2, toks, exps)
    assert np.array_equal(s["out"], full["out"][toks])
    assert np.array_equal(s["dx"], full["dx"][toks])
    for e in exps:
        assert np.array_equal(s["dW1"][e], full["dW1"][e])


@pytest.mark.parametrize("mutation", ["hp_not_quantised", "w2_wrong_axis", "dy_cols_as_rows"])
def test_wiring_mistakes_are_caught(mutation, monkeypatch):
    inp = _inp()
    ref = brute.mx_layer(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dout"], 2)
    if mutation == "hp_not_quantised":
        monkeypatch.setattr(oracle, "_gemm2_operand", lambda a, lib=None: np.asarray(a, np.float64))
    elif mutation == "w2_wrong_axis":
        real_w = oracle._mx_weights_bwd

        def fake_w(W1, W2, experts, lib=None):
            w1b, _ = real_w(W1, W2, experts, lib)
            return w1b, [oracle.mx_rows(W2[e]) if e in experts else None
                         for e in range(W2.shape[0])]
        monkeypatch.setattr(oracle, "_mx_weights_bwd", fake_w)
    else:
        real_c = oracle.mx_cols
        monkeypatch.setattr(oracle, "mx_cols", lambda a, lib=None: oracle.mx_rows(a, lib)
                            if np.asarray(a).shape[1] % 32 == 0 else real_c(a, lib))
    m = oracle.layer_mx(inp, 2)
    errs = [_rel(m["out"], ref["out"]), _rel(m["dx"], ref["dx"])] + \
           [_rel(m["dW1"][e], ref["dW1"][e]) for e in range(4)] + \
           [_rel(m["dW2"][e], ref["dW2"][e]) for e in range(4)]
    assert max(errs) > 2e-2, mutation


def test_expert_chunking_leaves_values_unchanged():
    """The MXFP8 layer takes its rows a few experts at a time (only those
    experts' dequantised weights are held): every chunk size gives the same
    bits, since each routed row depends only on its token and expert."""
    inp = _inp(T=60, d=64, E=6, k=3, h=32)
    r = oracle.route(inp["logits"], 3)
    rows = np.arange(60 * 3)
    lib = oracle.load()
    ref = oracle._mx_layer_rows(inp, 3, rows, r, lib, True, chunk=6)
    for chunk in (1, 4):
        got = oracle._mx_layer_rows(inp, 3, rows, r, lib, True, chunk=chunk)
        for key in ("ab", "hp", "y", "dy", "dab", "dx_perm"):
            assert np.array_equal(got[key], ref[key]), (chunk, key)
