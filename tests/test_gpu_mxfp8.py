"""GPU parity of the MXFP8 path against the oracle.

Quantised bytes (E4M3 elements, E8M0 scales) must be bit-exact given the same
input; GEMMs are fed the oracle's own quantised operands so each kernel is
checked in isolation; the MXFP8 layer is checked end to end and, at full
size, on sampled tokens and experts. Floating-point tolerance: 3e-2
(infinity-norm relative) for MXFP8 results; 1e-2 where only bf16 rounding of
identical fp8 products separates the two sides.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, dev, rel_fro, rel_inf, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routing_grouped_gemm_router_amd as moe


def _wide(shape, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape) * np.exp(rng.uniform(-12, 12, (shape[0], 1)))
    a[0, :32] = 0.0                       # an all-zero block
    a[1, 5] = 500.0                       # saturates
    a[2, :32] = 1e-41                     # fp32 subnormal block
    return a.astype(np.float32)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_quantise_rows_bit_exact(dt):
    a = _wide((257, 96), 1)
    x = dev(a, dt)
    q, s = moe.mxfp8_quantize(x, 1)
    qo, so = oracle.mxfp8_quantize(to_np(x), 1)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy(), so)


@pytest.mark.parametrize("groups", [[0, 300], [0, 1, 129, 129, 400, 401], [0, 0, 0, 77]])
def test_quantise_cols_grouped_bit_exact(groups):
    rows = groups[-1]
    a = _wide((max(rows, 3), 64), 2)[:rows]
    x = dev(a, torch.bfloat16)
    go = np.array(groups, np.int32)
    q, s = moe.mxfp8_quantize(x, 0, torch.from_numpy(go).cuda())
    qo, so = oracle.mxfp8_quantize(to_np(x), 0, go)
    assert np.array_equal(q.cpu().numpy()[:len(qo)], qo)
    assert np.array_equal(s.cpu().numpy()[:len(so)], so)


@pytest.mark.parametrize("dt,mapped", [(torch.bfloat16, False), (torch.bfloat16, True),
                                        (torch.float32, False)])
def test_quantise_cols_many_units(dt, mapped):
    """4096 x 4096 in 8 groups (an empty one, a one-row one): each workgroup of
    the column quantisers walks several 128-row units, with the next unit's
    tile (and, with a row map, its row indices) read ahead of the current
    one's encoding. Column layout bit-exact; the both-layout path too."""
    rows, cols = 4096, 4096
    a = synth.normal((rows, cols), 9, 0, 1.0)
    a[7, :32] = 0.0
    x = dev(a, dt)
    go = np.array([0, 300, 300, 1100, 2048, 2049, 3000, 3500, 4096], np.int32)
    g = torch.from_numpy(go).cuda()
    if mapped:
        perm = np.random.default_rng(4).integers(0, rows, rows).astype(np.int32)
        q, s = moe.mxfp8_quantize(x, 0, g, row_map=torch.from_numpy(perm).cuda())
        src = to_np(x)[perm]
    else:
        q, s = moe.mxfp8_quantize(x, 0, g)
        src = to_np(x)
    qo, so = oracle.mxfp8_quantize(src, 0, go)
    assert np.array_equal(q.cpu().numpy()[:len(qo)], qo)
    assert np.array_equal(s.cpu().numpy()[:len(so)], so)
    if not mapped:
        (q1, s1), (q0, s0) = moe.mxfp8_quantize_both(x, g)
        q1o, s1o = oracle.mxfp8_quantize(src, 1)
        assert np.array_equal(q0.cpu().numpy()[:len(qo)], qo)
        assert np.array_equal(s0.cpu().numpy()[:len(so)], so)
        assert np.array_equal(q1.cpu().numpy(), q1o) and np.array_equal(s1.cpu().numpy(), s1o)


def test_quantise_with_row_map():
    a = _wide((100, 128), 3)
    x = dev(a, torch.bfloat16)
    perm = np.random.default_rng(4).integers(0, 100, 250).astype(np.int32)
    go = np.array([0, 90, 90, 250], np.int32)
    q, s = moe.mxfp8_quantize(x, 0, torch.from_numpy(go).cuda(), row_map=torch.from_numpy(perm).cuda())
    qo, so = oracle.mxfp8_quantize(to_np(x)[perm], 0, go)
    assert np.array_equal(q.cpu().numpy()[:len(qo)], qo)
    assert np.array_equal(s.cpu().numpy()[:len(so)], so)
    q1, s1 = moe.mxfp8_quantize(x, 1, row_map=torch.from_numpy(perm).cuda())
    q1o, s1o = oracle.mxfp8_quantize(to_np(x)[perm], 1)
    assert np.array_equal(q1.cpu().numpy(), q1o) and np.array_equal(s1.cpu().numpy(), s1o)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_quantise_nan_elements(dt):
    """NaN elements (both signs) among finite ones: the block scale ignores
    them and each encodes as its sign | 0x7f, as the oracle does; a wave
    that holds a NaN takes the encoder's exact select path, the others the
    fast one, so blocks with and without NaN sit side by side."""
    x = dev(_wide((257, 160), 6), dt)
    # quiet NaNs of both signs, planted as bit patterns
    bits = x.view(torch.int32) if dt == torch.float32 else x.view(torch.int16)
    pos, neg = (0x7FC00000, -0x400000) if dt == torch.float32 else (0x7FC0, -0x40)
    bits[3, 7] = pos
    bits[3, 40] = neg
    bits[100, :32] = neg                  # a block of NaNs only
    bits[200, 150] = pos
    xn = to_np(x)
    assert np.isnan(xn[3, 7]) and not np.signbit(xn[3, 7])
    assert np.isnan(xn[3, 40]) and np.signbit(xn[3, 40])
    q, s = moe.mxfp8_quantize(x, 1)
    qo, so = oracle.mxfp8_quantize(xn, 1)
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)
    go = np.array([0, 5, 130, 257], np.int32)
    q0, s0 = moe.mxfp8_quantize(x, 0, torch.from_numpy(go).cuda())
    qo0, so0 = oracle.mxfp8_quantize(xn, 0, go)
    assert np.array_equal(q0.cpu().numpy()[:len(qo0)], qo0)
    assert np.array_equal(s0.cpu().numpy()[:len(so0)], so0)
    (qb1, sb1), (qb0, sb0) = moe.mxfp8_quantize_both(x, torch.from_numpy(go).cuda())
    assert np.array_equal(qb1.cpu().numpy(), qo) and np.array_equal(sb1.cpu().numpy(), so)
    assert np.array_equal(qb0.cpu().numpy()[:len(qo0)], qo0)
    assert np.array_equal(sb0.cpu().numpy()[:len(so0)], so0)


def test_permute_mxfp8_payload():
    T, d, E, k = 200, 256, 8, 3
    logits = synth.normal((T, E), 5, 0, 1.0)
    x = dev(synth.normal((T, d), 5, 1, 1.0), torch.bfloat16)
    xq, xs = moe.mxfp8_quantize(x, 1)
    r = moe.moe_route(dev(logits, torch.float32), k)
    xpq, xps = moe.moe_permute(xq, r["token_pos"], x_scale=xs)
    st = r["sorted_token"].long().cpu()
    assert torch.equal(xpq.cpu(), xq.cpu()[st]) and torch.equal(xps.cpu(), xs.cpu()[st])


# ---------------------------------------------------------------------------
# MXFP8 grouped GEMM, every role, on the oracle's quantised operands

def _deq_rows(q, s):
    return oracle.mxfp8_dequantize_rowwise(q, s)


@pytest.mark.parametrize("shape", [(300, 256, 8, 2, 128), (97, 128, 5, 3, 128)])
def test_mxfp8_gemm_stages(shape):
    T, d, E, k, h = shape
    R = T * k
    rng = np.random.default_rng(T)
    inp = dict(logits=synth.normal((T, E), 7, 0, 1.0),
               x=torch.from_numpy(synth.normal((T, d), 7, 1, 1.0)).bfloat16().float().numpy(),
               w1=synth.normal((E, 2 * h, d), 7, 2, 0.05), w2=synth.normal((E, d, h), 7, 3, 0.05))
    inp["logits"][:, 1] -= 100.0                      # an empty expert
    r = oracle.route(inp["logits"], k)
    off = r["offsets"]
    offd = torch.from_numpy(off).cuda()
    expert = oracle.expert_of_rows(r["counts"])
    x_perm = inp["x"][r["sorted_token"]]
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    W1, W2 = inp["w1"], inp["w2"]
    # forward weights (along d / h) and backward weights (per expert along 2h / d)
    w1q, w1s = oracle.mxfp8_quantize(W1.reshape(E * 2 * h, d), 1)
    w2q, w2s = oracle.mxfp8_quantize(W2.reshape(E * d, h), 1)
    w1tq, w1ts = oracle.mxfp8_quantize(W1.reshape(E * 2 * h, d), 0, np.arange(E + 1, dtype=np.int32) * 2 * h)
    w2tq, w2ts = oracle.mxfp8_quantize(W2.reshape(E * d, h), 0, np.arange(E + 1, dtype=np.int32) * d)
    W1f = _deq_rows(w1q, w1s).reshape(E, 2 * h, d)
    W2f = _deq_rows(w2q, w2s).reshape(E, d, h)
    W1b = np.stack([oracle.mx_cols(W1[e]) for e in range(E)])
    W2b = np.stack([oracle.mx_cols(W2[e]) for e in range(E)])
    bf = torch.bfloat16
    # GEMM1 + SwiGLU
    xq, xs = oracle.mxfp8_quantize(x_perm, 1)
    ab_ref, hp_ref, _ = oracle.rows_fwd(_deq_rows(xq, xs), expert, list(W1f), list(W2f), h, "bf16")
    ab = torch.empty((R, 2 * h), dtype=bf, device="cuda")
    hp = torch.empty((R, h), dtype=bf, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, u8(xq), u8(w1q), ab, offd, moe.MOE_EPI_SWIGLU_FWD,
                         N=2 * h, K=d, aux_out=hp, a_scale=u8(xs), b_scale=u8(w1s), dtype=moe.MOE_MXFP8)
    assert rel_inf(to_np(ab), ab_ref) <= TOL["bf16"]
    assert rel_inf(to_np(hp), hp_ref) <= TOL["bf16"]
    # GEMM2 on the oracle's quantised H'
    hq, hs = oracle.mxfp8_quantize(hp_ref, 1)
    _, _, y_ref = oracle.rows_fwd(_deq_rows(xq, xs), expert, list(W1f), list(W2f), h, "bf16",
                                  hp_in=_deq_rows(hq, hs))
    y = torch.empty((R, d), dtype=bf, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, u8(hq), u8(w2q), y, offd, N=d, K=h, a_scale=u8(hs),
                         b_scale=u8(w2s), dtype=moe.MOE_MXFP8)
    assert rel_inf(to_np(y), y_ref) <= TOL["bf16"]
    # GEMM2 dgrad + SwiGLU backward
    dy = torch.from_numpy(rng.standard_normal((R, d)).astype(np.float32)).bfloat16().float().numpy()
    dyq, dys = oracle.mxfp8_quantize(dy, 1)
    dab_ref, _ = oracle.rows_bwd(_deq_rows(dyq, dys), ab_ref, expert, list(W1b), list(W2b), h, "bf16")
    dab = torch.empty((R, 2 * h), dtype=bf, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_DGRAD, u8(dyq), u8(w2tq), dab, offd, moe.MOE_EPI_SWIGLU_BWD,
                         N=h, K=d, aux=dev(ab_ref, bf), a_scale=u8(dys), b_scale=u8(w2ts),
                         dtype=moe.MOE_MXFP8)
    assert rel_inf(to_np(dab), dab_ref) <= TOL["bf16"]
    # GEMM1 dgrad
    dq, ds = oracle.mxfp8_quantize(dab_ref, 1)
    _, dx_ref = oracle.rows_bwd(_deq_rows(dyq, dys), ab_ref, expert, list(W1b), list(W2b), h, "bf16",
                                dab_in=_deq_rows(dq, ds))
    dxp = torch.empty((R, d), dtype=bf, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_DGRAD, u8(dq), u8(w1tq), dxp, offd, N=d, K=2 * h,
                         a_scale=u8(ds), b_scale=u8(w1ts), dtype=moe.MOE_MXFP8)
    assert rel_inf(to_np(dxp), dx_ref) <= TOL["bf16"]
    # wgrads on column-block operands, in buffers of the size the library's
    # contract asks for (mxfp8_col_blocks blocks: the kernel may read a few
    # scale bytes past the last used block)
    nbw = moe.mxfp8_col_blocks(R, E)

    def sized(a, per_block):
        buf = np.zeros(nbw * per_block, np.uint8)
        buf[:a.size] = a.reshape(-1)
        return buf

    for (lhs, rhs, M, N) in ((dy, hp_ref, d, h), (dab_ref, x_perm, 2 * h, d)):
        aq, as_ = oracle.mxfp8_quantize(lhs, 0, off)
        bq, bs = oracle.mxfp8_quantize(rhs, 0, off)
        aq, as_ = sized(aq, 32 * M), sized(as_, M)
        bq, bs = sized(bq, 32 * N), sized(bs, N)
        dw = torch.full((E, M, N), float("nan"), device="cuda")
        moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, u8(aq), u8(bq), dw, offd, M=M, N=N,
                             a_scale=u8(as_), b_scale=u8(bs), dtype=moe.MOE_MXFP8, rows=R)
        for e in range(E):
            o0, o1 = off[e], off[e + 1]
            if o1 == o0:
                assert torch.all(dw[e] == 0)
                continue
            ref = oracle.wgrad(oracle.mx_cols(lhs[o0:o1]), oracle.mx_cols(rhs[o0:o1]))
            # identical fp8 products; the matrix core's 64-wide fp8 dot products
            # are not summed exactly in fp32 (measured ~1e-4), far inside 3e-2
            assert rel_inf(to_np(dw[e]), ref) <= 1e-3, e


# ---------------------------------------------------------------------------
# the MXFP8 layer

def _mx_inputs(T, d, E, k, h, seed):
    inp = dict(logits=synth.normal((T, E), seed, 0, 1.0), x=synth.normal((T, d), seed, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), seed, 2, 0.02),
               w2=synth.normal((E, d, h), seed, 3, 0.02), dout=synth.normal((T, d), seed, 4, 1.0))
    for key in ("x", "dout"):
        inp[key] = torch.from_numpy(inp[key]).bfloat16().float().numpy()
    return inp


def _run_mx(inp, k):
    layer = moe.MoELayerMX(dev(inp["w1"], torch.float32), dev(inp["w2"], torch.float32), k)
    out = layer.forward(dev(inp["x"], torch.bfloat16), dev(inp["logits"], torch.float32))
    g = layer.backward(dev(inp["dout"], torch.bfloat16))
    torch.cuda.synchronize()
    return layer, out, g


@pytest.mark.parametrize("shape", [(300, 256, 8, 2, 128), (130, 128, 16, 4, 128),
                                   # widest d, widest h; largest E with the largest k
                                   (64, 16384, 4, 2, 128), (64, 128, 4, 2, 8192),
                                   (2048, 128, 256, 8, 128)])
def test_mxfp8_layer_end_to_end(shape):
    T, d, E, k, h = shape
    inp = _mx_inputs(T, d, E, k, h, seed=11)
    m = oracle.layer_mx(inp, k)
    layer, out, g = _run_mx(inp, k)
    tol = TOL["mxfp8"]
    assert rel_inf(to_np(out), m["out"]) <= tol
    assert rel_inf(to_np(g["dx"]), m["dx"]) <= tol
    assert rel_inf(to_np(g["dlogits"]), m["dlogits"]) <= tol
    dw1, dw2 = to_np(g["dw1"]), to_np(g["dw2"])
    ref1 = np.stack([m["dW1"][e] for e in range(E)])
    ref2 = np.stack([m["dW2"][e] for e in range(E)])
    # each weight gradient as one tensor (the error metric of every other check)
    assert rel_inf(dw1, ref1) <= tol
    assert rel_inf(dw2, ref2) <= tol
    # and each expert's slice: the two sides quantise their own bf16 dAB and
    # dy, which differ by rounding in a few percent of the elements; where
    # that moves a value across an E4M3 rounding step (an eighth of it) or
    # changes a block's scale, one term of an expert's sum moves by up to
    # that much. The slice's largest such error against its largest value
    # grows with the number of slices checked (4 % at E = 256), so per
    # expert the relative Frobenius error is checked, and the infinity norm
    # with up to 16 experts
    for e in range(E):
        assert rel_fro(dw1[e], ref1[e]) <= tol, e
        assert rel_fro(dw2[e], ref2[e]) <= tol, e
        if E <= 16:
            assert rel_inf(dw1[e], ref1[e]) <= tol, e
            assert rel_inf(dw2[e], ref2[e]) <= tol, e


@pytest.mark.parametrize("case", ["one_hot", "two_hot"])
def test_mxfp8_hot_expert_split_wgrad(case):
    """The MXFP8 weight gradients' hot-expert path (an expert with more than
    twice the mean rows split over all XCDs; its 8- and 16-tile dW2 / dW1
    meet the split's condition) against the oracle, expert by expert."""
    T, d, E, k, h = 512, 1024, 8, 2, 256
    inp = _mx_inputs(T, d, E, k, h, seed=23)
    if case == "one_hot":           # every token's first choice is expert 3
        inp["logits"][:, 3] += 10.0
    else:                           # experts 2 and 5 take every token; the others none
        inp["logits"][:, 2] += 20.0
        inp["logits"][:, 5] += 10.0
    m = oracle.layer_mx(inp, k)
    counts = m["route"]["counts"]
    thresh = 2 * -(-(T * k) // E)
    assert [e for e in range(E) if counts[e] > thresh] == ([3] if case == "one_hot" else [2, 5])
    layer, out, g = _run_mx(inp, k)
    tol = TOL["mxfp8"]
    assert rel_inf(to_np(out), m["out"]) <= tol
    assert rel_inf(to_np(g["dx"]), m["dx"]) <= tol
    assert rel_inf(to_np(g["dlogits"]), m["dlogits"]) <= tol
    dw1, dw2 = to_np(g["dw1"]), to_np(g["dw2"])
    for e in range(E):
        if counts[e] == 0:
            assert np.all(dw1[e] == 0) and np.all(dw2[e] == 0), e
            continue
        assert rel_inf(dw1[e], m["dW1"][e]) <= tol, e
        assert rel_inf(dw2[e], m["dW2"][e]) <= tol, e


@pytest.mark.parametrize("shape,empty", [((1, 128, 1, 1, 128), None),    # one token, one expert
                                         ((3, 128, 8, 8, 128), None),    # k = E
                                         ((200, 256, 6, 2, 128), -1),    # last expert empty
                                         ((200, 128, 6, 2, 256), 0)])    # first expert empty
def test_mxfp8_layer_edge_cases(shape, empty):
    T, d, E, k, h = shape
    inp = _mx_inputs(T, d, E, k, h, seed=5)
    if empty is not None:
        inp["logits"][:, empty] -= 100.0
    m = oracle.layer_mx(inp, k)
    layer, out, g = _run_mx(inp, k)
    tol = TOL["mxfp8"]
    assert rel_inf(to_np(out), m["out"]) <= tol
    assert rel_inf(to_np(g["dx"]), m["dx"]) <= tol
    assert rel_inf(to_np(g["dlogits"]), m["dlogits"]) <= tol
    assert rel_inf(to_np(g["dw1"]), np.stack([m["dW1"][e] for e in range(E)])) <= tol
    assert rel_inf(to_np(g["dw2"]), np.stack([m["dW2"][e] for e in range(E)])) <= tol
    if empty is not None:
        assert torch.all(g["dw1"][empty] == 0) and torch.all(g["dw2"][empty] == 0)


@pytest.mark.parametrize("shape", [(300, 256, 8, 2, 128), (200, 128, 8, 2, 512)])   # h < d, h > d
def test_mxfp8_recompute_matches_saved(shape):
    """recompute=True re-quantises and re-dispatches x and reruns GEMM1 in
    the backward: bit-identical gradients to the layer that keeps A||B and H'."""
    T, d, E, k, h = shape
    inp = _mx_inputs(T, d, E, k, h, seed=17)
    base, out0, g0 = _run_mx(inp, k)
    out0 = out0.clone()
    g0 = {key: v.clone() for key, v in g0.items() if v is not None and not key.startswith("_")}
    layer = moe.MoELayerMX(dev(inp["w1"], torch.float32), dev(inp["w2"], torch.float32), k,
                           recompute=True)
    out = layer.forward(dev(inp["x"], torch.bfloat16), dev(inp["logits"], torch.float32))
    torch.cuda.synchronize()
    for t in moe._SCRATCH.values():
        t.fill_(float("nan") if t.is_floating_point() else 0x7F)
    g = layer.backward(dev(inp["dout"], torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(out, out0)
    for key in ("dx", "dw1", "dw2", "dlogits"):
        assert torch.equal(g[key], g0[key]), key
    assert layer.held_bytes() < base.held_bytes()


@pytest.mark.timeout(900)
def test_mxfp8_full_size_sampled():
    """The 32768-token, d=4096, E=128, h=2048 workload in the launch
    configuration the bench times: 256 sampled tokens (out, dX, dlogits) and
    the weight gradients of the hottest, a median and three random experts."""
    w = synth.WORKLOADS["e128_mxfp8"]
    d_in = synth.device_inputs(w, seed=0)
    layer = moe.MoELayerMX(d_in["w1"], d_in["w2"], w.k)
    out = layer.forward(d_in["x"], d_in["logits"])
    g = layer.backward(d_in["dout"])
    torch.cuda.synchronize()
    counts = layer.route["counts"].cpu().numpy()
    toks = synth.sample_indices(w.T, 256, seed=5)
    nz = np.flatnonzero(counts)
    hot = int(np.argmax(counts))
    med = int(nz[np.argsort(counts[nz], kind="stable")[len(nz) // 2]])
    rest = np.array(sorted(set(nz.tolist()) - {hot, med}))
    exps = sorted({hot, med} | {int(rest[i]) for i in synth.sample_indices(len(rest), 3, seed=6)})
    idx = layer.route["topk_idx"].cpu().numpy()
    needed = sorted(set(idx[toks].reshape(-1).tolist()) | set(exps))
    # host copies of only the inputs the sample needs
    host = dict(logits=to_np(d_in["logits"]), x=to_np(d_in["x"]), dout=to_np(d_in["dout"]))
    E = w.E
    w1 = np.zeros((E, 2 * w.h, w.d), np.float32)
    w2 = np.zeros((E, w.d, w.h), np.float32)
    for e in needed:
        w1[e] = to_np(d_in["w1"][e])
        w2[e] = to_np(d_in["w2"][e])
    host.update(w1=w1, w2=w2)
    m = oracle.layer_mx(host, w.k, toks, exps, progress=lambda msg: print(msg, flush=True))
    assert np.array_equal(m["route"]["counts"], counts)
    tol = TOL["mxfp8"]
    assert rel_inf(to_np(out)[toks], m["out"]) <= tol
    assert rel_inf(to_np(g["dx"])[toks], m["dx"]) <= tol
    assert rel_inf(to_np(g["dlogits"])[toks], m["dlogits"]) <= tol
    # weight gradients with E = 128: each expert's slice by the relative
    # Frobenius norm, as in the end-to-end check with more than 16 experts.
    # Each side quantises its own bf16 dAB and dy, which differ by one bf16
    # rounding in a few percent of the elements (the matrix core's fp8 dot
    # products are not summed exactly in fp32); where that moves a value
    # across an E4M3 step, one term of an expert's sum moves by up to an
    # eighth, so a slice's infinity norm can reach the tolerance while its
    # Frobenius error stays far below it. The infinity norms are printed.
    for e in exps:
        g1, g2 = to_np(g["dw1"][e]), to_np(g["dw2"][e])
        f1, f2 = rel_fro(g1, m["dW1"][e]), rel_fro(g2, m["dW2"][e])
        print(f"expert {e} rows {counts[e]}: dW1 fro {f1:.2e} inf {rel_inf(g1, m['dW1'][e]):.2e}; "
              f"dW2 fro {f2:.2e} inf {rel_inf(g2, m['dW2'][e]):.2e}", flush=True)
        assert f1 <= tol and f2 <= tol, e


def test_mxfp8_backward_forms_dy_bit_exact():
    """The MXFP8 backward forms dy_perm inside its quantiser from the dOut rows
    and each routed row's gate, without storing it. Its dAB and dW2 must equal,
    bit for bit, the same MXFP8 GEMMs run on dy_perm as the bf16 combine
    backward stores it (bf16 layer on the same routing and dOut), quantised
    by mxfp8_quantize_both, with the MXFP8 layer's own saved a, b and H'
    (the column layout of H' that its GEMM1 stored)."""
    T, d, E, k, h = 300, 256, 8, 2, 128
    inp = _mx_inputs(T, d, E, k, h, seed=11)
    inp["logits"][:, 1] -= 100.0                      # an empty expert
    layer, _, g = _run_mx(inp, k)
    off = layer.route["offsets"]
    R = T * k
    # dy_perm rows as the combine backward stores them (independent of the
    # weights): the bf16 layer on the same logits and dOut
    lb = moe.MoELayer(dev(inp["w1"], torch.bfloat16), dev(inp["w2"], torch.bfloat16), k)
    lb.forward(dev(inp["x"], torch.bfloat16), dev(inp["logits"], torch.float32))
    gb = lb.backward(dev(inp["dout"], torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(lb.route["offsets"], off) and torch.equal(lb.route["token_pos"], layer.route["token_pos"])
    (dyq, dys), (dyc, dycs) = moe.mxfp8_quantize_both(gb["dy_perm"], off)
    # GEMM2 dgrad + SwiGLU backward on the rows layout
    dab = torch.empty((R, 2 * h), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_DGRAD, dyq, layer.w2t, dab, off, moe.MOE_EPI_SWIGLU_BWD,
                         N=h, K=d, aux=layer.ab, a_scale=dys, b_scale=layer.w2ts,
                         dtype=moe.MOE_MXFP8)
    assert torch.equal(dab, g["dab"])
    # GEMM2 wgrad on the column layouts of dy and H'
    hc, hcs = layer.hpc, layer.hpcs
    dw2 = torch.full((E, d, h), float("nan"), device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, dyc, hc, dw2, off, M=d, N=h, a_scale=dycs,
                         b_scale=hcs, dtype=moe.MOE_MXFP8, rows=R)
    torch.cuda.synchronize()
    assert torch.equal(dw2, g["dw2"])


def test_mxfp8_backward_with_forward_quantised_hp_bit_exact():
    """The MXFP8 layer quantises H' in both layouts in the forward and hands
    the backward H' along rows per expert (hp_cols), so the backward reads no
    bf16 H'. The gradients equal, bit for bit, those of the backward that
    quantises the bf16 H' itself."""
    T, d, E, k, h = 300, 256, 8, 2, 128
    inp = _mx_inputs(T, d, E, k, h, seed=12)
    inp["logits"][:, 1] -= 100.0                      # an empty expert
    layer, _, g = _run_mx(inp, k)
    assert layer.saved().get("hp_cols") is not None and layer.saved()["hp"] is None
    # the same forward again with H' stored in bf16 (and quantised by its own
    # pass), for the backward that quantises bf16 H' itself
    layer.fuse_hp = False
    layer.forward(dev(inp["x"], torch.bfloat16), dev(inp["logits"], torch.float32))
    sv = layer.saved()
    sv.update(hp=layer.hp, hp_cols=None, hp_cols_scale=None)
    g2 = moe.moe_backward(sv, dev(inp["dout"], torch.bfloat16), E, k, d, h, mxfp8=True)
    torch.cuda.synchronize()
    for key in ("dx", "dlogits", "dw1", "dw2", "dab", "dx_perm", "dgate"):
        assert torch.equal(g[key], g2[key]), key


def _gemm1_mx_operands(T, d, E, k, h, seed, starve=()):
    inp = _mx_inputs(T, d, E, k, h, seed)
    for e in starve:
        inp["logits"][:, e] -= 100.0                  # no rows for expert e
    r = oracle.route(inp["logits"], k)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xq, xs = oracle.mxfp8_quantize(inp["x"][r["sorted_token"]], 1)
    w1q, w1s = oracle.mxfp8_quantize(inp["w1"].reshape(E * 2 * h, d), 1)
    return r, u8(xq), u8(xs), u8(w1q), u8(w1s), torch.from_numpy(r["offsets"]).cuda()


# (T, d, E, k, h): an empty expert among ragged groups; h = 160, whose second
# n-tile holds 32 hidden units (waves past h store nothing); groups of ~10
# rows, where whole waves of a 128-row unit are column-layout padding; one
# expert; the largest E
@pytest.mark.parametrize("shape,starve", [((300, 256, 8, 2, 128), (1,)),
                                          ((97, 128, 5, 3, 160), ()),
                                          ((40, 128, 8, 2, 128), (0, 7)),
                                          ((200, 128, 1, 1, 64), ()),
                                          ((600, 128, 256, 4, 96), ())])
def test_gemm1_quantised_hp_equals_quantiser(shape, starve):
    """The MXFP8 SwiGLU forward that stores H' quantised writes A||B and both
    MXFP8 layouts of H' byte for byte as the plain epilogue followed by the
    both-layout quantiser on its bf16 H' (every byte of the output buffers,
    pre-filled alike, so padding and untouched bytes are compared too)."""
    T, d, E, k, h = shape
    R = T * k
    r, xq, xs, w1q, w1s, offd = _gemm1_mx_operands(T, d, E, k, h, seed=31, starve=starve)
    assert all(r["counts"][e] == 0 for e in starve)
    nb = moe.mxfp8_col_blocks(R, E)
    bf = torch.bfloat16
    kw = dict(N=2 * h, K=d, a_scale=xs, b_scale=w1s, dtype=moe.MOE_MXFP8)
    ab_ref = torch.full((R, 2 * h), 3.0, dtype=bf, device="cuda")
    hp = torch.empty((R, h), dtype=bf, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, xq, w1q, ab_ref, offd, moe.MOE_EPI_SWIGLU_FWD,
                         aux_out=hp, **kw)
    fill = lambda *shape: torch.full(shape, 0x5A, dtype=torch.uint8, device="cuda")
    ref = (fill(R, h), fill(R, h // 32), fill(nb * 32 * h), fill(nb * h))
    moe.mxfp8_quantize_both(hp, offd, out=ref)
    ab = torch.full((R, 2 * h), 3.0, dtype=bf, device="cuda")
    got = (fill(R, h), fill(R, h // 32), fill(nb * 32 * h), fill(nb * h))
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, xq, w1q, ab, offd, moe.MOE_EPI_SWIGLU_FWD,
                         aux_out=got[0], aux_out_scale=got[1], aux_out_cols=got[2],
                         aux_out_cols_scale=got[3], **kw)
    torch.cuda.synchronize()
    assert torch.equal(ab, ab_ref)
    for name, a, b in zip(("rows", "row scales", "cols", "col scales"), got, ref):
        diff = torch.nonzero(a != b)
        assert diff.numel() == 0, (name, diff[:8].flatten().tolist())


# the layer needs h % 128 == 0 (GEMM2's MXFP8 reduction); groups of ~32 rows
# leave whole waves of padding in each 128-row unit
@pytest.mark.parametrize("shape", [(300, 256, 8, 2, 128), (130, 128, 16, 4, 256)])
def test_mxfp8_layer_quantised_hp_matches_separate_pass(shape):
    """The MXFP8 layer with H' quantised in GEMM1's epilogue gives the same
    output and gradients, bit for bit, as with bf16 H' and a separate
    quantiser pass."""
    T, d, E, k, h = shape
    inp = _mx_inputs(T, d, E, k, h, seed=17)
    inp["logits"][:, 2] -= 100.0                      # an empty expert
    layer, out, g = _run_mx(inp, k)
    out, g = out.clone(), {key: v.clone() for key, v in g.items() if v is not None}
    layer.fuse_hp = False
    out2 = layer.forward(dev(inp["x"], torch.bfloat16), dev(inp["logits"], torch.float32))
    g2 = layer.backward(dev(inp["dout"], torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for key in ("dx", "dlogits", "dw1", "dw2", "dgate"):
        assert torch.equal(g[key], g2[key]), key
