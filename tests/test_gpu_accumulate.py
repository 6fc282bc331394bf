"""Gradient accumulation and the fused weight re-quantisation on the GPU.

WGRAD with accumulate adds its product to C with one fp32 add per element,
so it must equal C0 + (the overwriting WGRAD's result) exactly, leave the
weight gradient of an expert with no rows untouched, and stay within the
dtype's tolerance of C0 + the oracle's weight gradient. mxfp8_quantize_both
must write exactly the bytes of mxfp8_quantize along each axis."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, dev, rel_inf, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routing_grouped_gemm_router_amd as moe


def _groups(R, E, seed):
    """Uneven groups with an empty one (expert 1) and a one-row one (expert 2)."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 3 * R // E, E)
    c[1], c[2] = 0, 1
    c[0] += R - c.sum()
    assert c[0] >= 0
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int32)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_wgrad_accumulate(dt):
    R, E, M, N = 700, 6, 96, 160
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    off = _groups(R, E, 1)
    a = synth.normal((R, M), 1, 0, 1.0)
    b = synth.normal((R, N), 1, 1, 1.0)
    if dt == "bf16":
        a = torch.from_numpy(a).bfloat16().float().numpy()
        b = torch.from_numpy(b).bfloat16().float().numpy()
    offd = torch.from_numpy(off).cuda()
    c0 = torch.randn(E, M, N, device="cuda")
    over = torch.full((E, M, N), float("nan"), device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, dev(a, tdt), dev(b, tdt), over, offd, M=M, N=N)
    acc = c0.clone()
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, dev(a, tdt), dev(b, tdt), acc, offd, M=M, N=N,
                         accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc, c0 + over)
    assert torch.equal(acc[1], c0[1])                      # no rows: unchanged
    for e in range(E):
        ref = to_np(c0[e]).astype(np.float64) + oracle.wgrad(a[off[e]:off[e + 1]], b[off[e]:off[e + 1]]) \
            if off[e + 1] > off[e] else to_np(c0[e])
        assert rel_inf(to_np(acc[e]), ref) <= TOL[dt], e


def test_wgrad_accumulate_mxfp8():
    R, E, M, N = 640, 5, 128, 256
    off = _groups(R, E, 2)
    offd = torch.from_numpy(off).cuda()
    a = torch.from_numpy(synth.normal((R, M), 2, 0, 1.0)).bfloat16().cuda()
    b = torch.from_numpy(synth.normal((R, N), 2, 1, 1.0)).bfloat16().cuda()
    aq, as_ = moe.mxfp8_quantize(a, 0, offd)
    bq, bs = moe.mxfp8_quantize(b, 0, offd)
    c0 = torch.randn(E, M, N, device="cuda")
    over = torch.full((E, M, N), float("nan"), device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, aq, bq, over, offd, M=M, N=N, a_scale=as_,
                         b_scale=bs, dtype=moe.MOE_MXFP8, rows=R)
    acc = c0.clone()
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, aq, bq, acc, offd, M=M, N=N, a_scale=as_,
                         b_scale=bs, dtype=moe.MOE_MXFP8, accumulate=True, rows=R)
    torch.cuda.synchronize()
    assert torch.equal(acc, c0 + over)
    assert torch.equal(acc[1], c0[1])


def _layer_in(T, d, E, k, h, seed):
    inp = dict(logits=synth.normal((T, E), seed, 0, 1.0), x=synth.normal((T, d), seed, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), seed, 2, 0.05),
               w2=synth.normal((E, d, h), seed, 3, 0.05), dout=synth.normal((T, d), seed, 4, 1.0))
    return inp


@pytest.mark.parametrize("shape", [(256, 128, 8, 2, 128), (200, 128, 8, 2, 512)])   # h = d, h > d
@pytest.mark.parametrize("mx", [False, True])
def test_layer_accumulates_over_micro_batches(mx, shape):
    """Two micro-batches: the second backward with accumulate_dw adds its
    weight gradients to the first's, exactly (one fp32 add per element)."""
    T, d, E, k, h = shape
    a = _layer_in(T, d, E, k, h, 21)
    b = _layer_in(T, d, E, k, h, 22)
    w1 = dev(a["w1"], torch.float32 if mx else torch.bfloat16)
    w2 = dev(a["w2"], torch.float32 if mx else torch.bfloat16)
    make = (lambda: moe.MoELayerMX(w1, w2, k)) if mx else (lambda: moe.MoELayer(w1, w2, k))
    bf = torch.bfloat16

    def run(layer, inp, acc=False):
        layer.forward(dev(inp["x"], bf), dev(inp["logits"], torch.float32))
        return layer.backward(dev(inp["dout"], bf), accumulate_dw=acc)

    l1 = make()
    g1 = {n: run(l1, a)[n].clone() for n in ("dw1", "dw2")}
    l2 = make()
    g2 = {n: run(l2, b)[n].clone() for n in ("dw1", "dw2")}
    l3 = make()
    run(l3, a)
    g3 = run(l3, b, acc=True)
    torch.cuda.synchronize()
    for n in ("dw1", "dw2"):
        assert torch.equal(g3[n], g1[n] + g2[n]), n


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [320, 256, 96])   # a partial last column tile / whole tiles only / one partial tile
def test_quantize_both_matches_separate(dt, cols):
    rows = 8 * 192
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = torch.from_numpy(synth.normal((rows, cols), 4, 0, 0.02)).to(tdt).cuda()
    x[5, :40] = 0.0                                        # an all-zero block
    groups = torch.arange(0, 9, dtype=torch.int32, device="cuda") * 192
    (q1, s1), (q0, s0) = moe.mxfp8_quantize_both(x, groups)
    r1, rs1 = moe.mxfp8_quantize(x, 1)
    r0, rs0 = moe.mxfp8_quantize(x, 0, groups)
    torch.cuda.synchronize()
    assert torch.equal(q1, r1) and torch.equal(s1, rs1)
    n = 8 * 2 * 4 * 32 * cols     # 8 groups of 2 units of 128 rows (192 padded to 256): the bytes written
    assert torch.equal(q0[:n], r0[:n]) and torch.equal(s0[:n // 32], rs0[:n // 32])
    # and against the oracle along rows
    oq, os_ = oracle.mxfp8_quantize(to_np(x), 1)
    assert np.array_equal(to_np(q1), oq) and np.array_equal(to_np(s1), os_)


def test_quantize_both_unaligned_row_scales():
    """Row-layout scales at an odd address: the kernel's per-row word stores
    of four scale bytes must give way to byte stores."""
    import ctypes
    rows, cols = 8 * 192, 256
    x = torch.from_numpy(synth.normal((rows, cols), 5, 0, 0.02)).to(torch.bfloat16).cuda()
    groups = torch.arange(0, 9, dtype=torch.int32, device="cuda") * 192
    (r1, rs1), (r0, rs0) = moe.mxfp8_quantize_both(x, groups)
    q1 = torch.empty_like(r1)
    s1_buf = torch.full((rs1.numel() + 1,), 0xA5, dtype=torch.uint8, device="cuda")
    q0 = torch.empty_like(r0)
    s0 = torch.empty_like(rs0)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    st = moe.lib().mxfp8_quantize_both(P(x), 1, rows, cols, P(groups), 8, P(q1), P(s1_buf, 1), P(q0), P(s0),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(q1, r1)
    assert torch.equal(s1_buf[1:].view(rs1.shape), rs1)
    assert s1_buf[0].item() == 0xA5                    # nothing written before the array
    n = 8 * 2 * 4 * 32 * cols
    assert torch.equal(q0[:n], r0[:n]) and torch.equal(s0[:n // 32], rs0[:n // 32])
