"""GPU parity of moe_load_balance against the oracle's load_balance.

Statistics derived from the integer counts (max / min load over the mean,
coefficient of variation, empty experts) are exact up to fp32 output
rounding; the probability-based ones are fp32 softmax sums over T tokens,
checked to 1e-4 relative; the gradient to 1e-5 of its largest element (plus a floor of 1e-6 of its
bound alpha E / T, for the cases where it is exactly zero). The
gradient is added into dlogits, so it is checked on top of a random base."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev, rel_inf, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routing_grouped_gemm_router_amd as moe


def _check(logits_np, k, alpha, zipf=False):
    T, E = logits_np.shape
    r = oracle.route(logits_np, k)
    ref_st, ref_g = oracle.load_balance(logits_np, r["counts"], k, alpha)
    logits = dev(logits_np, torch.float32)
    counts = torch.from_numpy(r["counts"].astype(np.int32)).cuda()
    dl0 = torch.zeros(T, E, device="cuda")
    st = moe.moe_load_balance(logits, counts, k, alpha, dlogits=dl0)
    st2 = moe.moe_load_balance(logits, counts, k, alpha)
    gen = torch.Generator(device="cuda").manual_seed(T * 1000 + E)
    base = torch.randn(T, E, device="cuda", generator=gen)
    dlb = base.clone()
    moe.moe_load_balance(logits, counts, k, alpha, dlogits=dlb)
    torch.cuda.synchronize()
    st, st2 = to_np(st), to_np(st2)
    assert np.array_equal(st, st2)                          # deterministic, dlogits or not
    for i in (0, 1, 2, 3):
        assert st[i] == pytest.approx(ref_st[i], rel=1e-4), oracle.LB_STATS[i]
    for i in (4, 5, 6):
        assert st[i] == pytest.approx(ref_st[i], rel=1e-6, abs=1e-7), oracle.LB_STATS[i]
    assert st[7] == ref_st[7]
    if T:
        g = to_np(dl0)
        # |dL/dl| <= alpha E / T: a millionth of that bound is the floor where
        # the exact gradient vanishes (k = E: every f_e = 1/E)
        floor = 1e-6 * alpha * E / T
        assert np.abs(g - ref_g).max() <= 1e-5 * np.abs(ref_g).max() + floor
        # added, not overwritten: base + g up to the rounding of one fp32 add.
        # The kernel may fuse the gradient's last product into the add, which
        # skips g's own rounding: where base and g nearly cancel, the sum can
        # then differ from base + g by up to one ulp of g, far more than an
        # ulp of the small sum
        want = (to_np(base) + g).astype(np.float32)
        tol = np.spacing(np.abs(want)) + np.spacing(np.abs(g))
        assert np.all(np.abs(to_np(dlb) - want) <= tol)


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (300, 100, 3), (513, 128, 4), (64, 256, 8),
                                   (1000, 64, 1), (37, 5, 5)])
def test_load_balance_parity(T, E, k):
    logits = synth.normal((T, E), 3, 0, 1.0)
    _check(logits, k, alpha=0.01)


def test_load_balance_skewed():
    """Zipf-skewed routing: the hard-load statistics far from uniform."""
    w = synth.WORKLOADS["e128_bf16_zipf"]
    logits = synth.normal((4096, w.E), 0, synth.STREAM_LOGITS, 1.0) + \
        synth.zipf_bias(w.E, w.zipf_s)[None, :]
    _check(logits.astype(np.float32), w.k, alpha=0.01)


def test_load_balance_full_size():
    w = synth.WORKLOADS["e128_bf16"]
    d_in = synth.device_inputs(w, seed=0, with_dout=False)
    logits_np = to_np(d_in["logits"])
    _check(logits_np, w.k, alpha=0.001)


def test_load_balance_zero_tokens():
    st = moe.moe_load_balance(torch.empty((0, 8), device="cuda"),
                              torch.zeros(8, dtype=torch.int32, device="cuda"), 2, 1.0)
    torch.cuda.synchronize()
    assert torch.all(st == 0)


def test_layer_with_balancing_loss():
    """MoELayer(aux_alpha=...): the layer's logit gradient plus the balancing
    loss gradient, and the statistics of the forward's routing."""
    T, d, E, k, h, alpha = 300, 128, 16, 2, 64, 0.05
    inp = dict(logits=synth.normal((T, E), 5, 0, 1.0), x=synth.normal((T, d), 5, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), 5, 2, 0.05), w2=synth.normal((E, d, h), 5, 3, 0.05),
               dout=synth.normal((T, d), 5, 4, 1.0))
    args = [dev(inp[n], torch.float32) for n in ("w1", "w2")]
    plain = moe.MoELayer(*args, k)
    plain.forward(dev(inp["x"], torch.float32), dev(inp["logits"], torch.float32))
    d0 = plain.backward(dev(inp["dout"], torch.float32))["dlogits"].clone()
    layer = moe.MoELayer(*args, k, aux_alpha=alpha)
    layer.forward(dev(inp["x"], torch.float32), dev(inp["logits"], torch.float32))
    st = to_np(layer.lb_stats).copy()
    d1 = layer.backward(dev(inp["dout"], torch.float32))["dlogits"]
    torch.cuda.synchronize()
    r = oracle.route(inp["logits"], k)
    ref_st, ref_g = oracle.load_balance(inp["logits"], r["counts"], k, alpha)
    assert st[0] == pytest.approx(ref_st[0], rel=1e-4)
    assert st[7] == ref_st[7]
    diff = to_np(d1).astype(np.float64) - to_np(d0)
    assert np.abs(diff - ref_g).max() <= 1e-4 * np.abs(ref_g).max() + \
        np.spacing(np.abs(to_np(d1))).max()
