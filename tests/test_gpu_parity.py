"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (routing indices, counts, offsets, positions, permuted rows,
MXFP8 bytes) must be bit-exact; floating-point outputs must be within the
infinity-norm relative error 1e-2 for bf16 and 1e-4 for fp32. Each kernel is
first checked in isolation on the oracle's own inputs, then the whole layer
end to end.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, dev, rel_inf, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routing_grouped_gemm_router_amd as moe


def _route_eq(g, o):
    for key in ("topk_idx", "counts", "offsets", "tile_offsets", "token_pos", "sorted_token",
                "sorted_slot"):
        a = g[key].cpu().numpy()
        assert np.array_equal(a, o[key]), key
    gg = g["topk_gate"].cpu().numpy()
    if gg.size:
        assert np.abs(gg - o["topk_gate"]).max() <= 1e-6


def test_single_hip_runtime():
    """libmoe binds to the HIP runtime torch already loaded (one libamdhip64)."""
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths
    assert any("libmoe.so" in l for l in maps.splitlines())


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (300, 16, 3), (1000, 128, 4), (64, 256, 8),
                                   (65, 5, 1), (1, 4, 4), (0, 8, 2), (777, 33, 5)])
def test_route_bit_exact(T, E, k):
    logits = synth.normal((T, E), 3, 0, 1.0)
    g = moe.moe_route(dev(logits, torch.float32), k, tile_m=64)
    torch.cuda.synchronize()
    _route_eq(g, oracle.route(logits, k, 64))


def test_route_ties_and_signed_zero():
    rows = np.array(np.meshgrid(*[[-0.0, 0.0, 1.0]] * 4)).reshape(4, -1).T.astype(np.float32)
    rows = np.concatenate([rows] * 3)       # several chunks, ties across them
    for k in (1, 2, 3, 4):
        g = moe.moe_route(dev(rows, torch.float32), k, tile_m=7)
        torch.cuda.synchronize()
        _route_eq(g, oracle.route(rows, k, 7))


@pytest.mark.parametrize("name", ["e128_bf16", "e128_bf16_zipf", "e8_bf16_fwd", "e16_bf16_ep_share"])
def test_route_full_size(name):
    w = synth.WORKLOADS[name]
    logits = synth.normal((w.T, w.E), 0, synth.STREAM_LOGITS, w.logit_scale)
    if w.zipf_s:
        logits = logits + synth.zipf_bias(w.E, w.zipf_s)
    g = moe.moe_route(dev(logits, torch.float32), w.k)
    torch.cuda.synchronize()
    _route_eq(g, oracle.route(logits, w.k, 128))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permute_bit_exact(dtype):
    T, d, E, k = 333, 256, 8, 3
    logits = synth.normal((T, E), 1, 0, 1.0)
    x = synth.normal((T, d), 1, 1, 1.0)
    xd = dev(x, dtype)
    r = moe.moe_route(dev(logits, torch.float32), k)
    xp = moe.moe_permute(xd, r["token_pos"])
    torch.cuda.synchronize()
    st = r["sorted_token"].cpu().numpy()
    assert torch.equal(xp.cpu(), xd.cpu()[torch.from_numpy(st).long()])


def _layer_inputs(T, d, E, k, h, seed=0, dt="bf16"):
    inp = dict(logits=synth.normal((T, E), seed, 0, 1.0), x=synth.normal((T, d), seed, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), seed, 2, 0.05),
               w2=synth.normal((E, d, h), seed, 3, 0.05), dout=synth.normal((T, d), seed, 4, 1.0))
    if dt == "bf16":
        for key in ("x", "w1", "w2", "dout"):
            inp[key] = torch.from_numpy(inp[key]).bfloat16().float().numpy()
    return inp


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_combine(dt):
    T, d, E, k, h = 300, 256, 8, 3, 64
    inp = _layer_inputs(T, d, E, k, h, dt=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    o = oracle.route(inp["logits"], k)
    y = synth.normal((T * k, d), 2, 9, 1.0)
    if dt == "bf16":
        y = torch.from_numpy(y).bfloat16().float().numpy()
    out = moe.moe_combine(dev(y, tdt), dev(o["topk_gate"], torch.float32),
                          torch.from_numpy(o["token_pos"]).cuda())
    ref = oracle.combine(o["topk_gate"], o["token_pos"], y, dt)
    assert rel_inf(to_np(out), ref) <= TOL[dt] / 10


# ---------------------------------------------------------------------------
# grouped GEMM, stage by stage on the oracle's inputs

SHAPES = [  # T, d, E, k, h: several tiles plus ragged tails, an empty expert
    (300, 256, 8, 2, 192),
    (513, 128, 5, 3, 320),
    (64, 96, 3, 1, 32),
    # d % 64 == 32: GEMM2 dgrad's last K step is half a step, the weight rows
    # past K must not be read (the last expert's W2 ends there)
    (97, 32, 3, 3, 1024),
    (333, 96, 7, 3, 160),
    # the most experts the library takes: the fp32 kernel's 256-thread
    # workgroups load all 257 offsets (expert 1 empty, as below)
    (400, 64, 256, 5, 96),
]


def _stage_data(T, d, E, k, h, dt):
    inp = _layer_inputs(T, d, E, k, h, seed=T, dt=dt)
    if E >= 5:
        inp["logits"][:, 1] -= 100.0        # expert 1 gets no rows
    f = oracle.layer_forward(inp, k, dt)
    b = oracle.layer_backward(inp, f, k, dt)
    return inp, f, b


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gemm_stages(shape, dt):
    T, d, E, k, h = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp, f, b = _stage_data(T, d, E, k, h, dt)
    R = T * k
    off = torch.from_numpy(f["route"]["offsets"]).cuda()
    w1 = dev(inp["w1"], tdt)
    w2 = dev(inp["w2"], tdt)
    tol = TOL[dt]
    # GEMM1 + SwiGLU
    xp = dev(f["x_perm"], tdt)
    ab = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    hp = torch.empty((R, h), dtype=tdt, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, xp, w1, ab, off, moe.MOE_EPI_SWIGLU_FWD, N=2 * h, K=d,
                         aux_out=hp)
    assert rel_inf(to_np(ab), f["ab"]) <= tol
    assert rel_inf(to_np(hp), f["hp"]) <= tol
    # GEMM2 on the oracle's H'
    y = torch.empty((R, d), dtype=tdt, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_FWD, dev(f["hp"], tdt), w2, y, off, N=d, K=h)
    assert rel_inf(to_np(y), f["y_perm"]) <= tol
    # GEMM2 dgrad + SwiGLU backward on the oracle's dy, AB
    dab = torch.empty((R, 2 * h), dtype=tdt, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_DGRAD, dev(b["dy_perm"], tdt), w2, dab, off,
                         moe.MOE_EPI_SWIGLU_BWD, N=h, K=d, aux=dev(f["ab"], tdt))
    assert rel_inf(to_np(dab), b["dab"]) <= tol
    # GEMM1 dgrad on the oracle's dAB
    dxp = torch.empty((R, d), dtype=tdt, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_DGRAD, dev(b["dab"], tdt), w1, dxp, off, N=d, K=2 * h)
    assert rel_inf(to_np(dxp), b["dx_perm"]) <= tol
    # wgrads
    dw2 = torch.full((E, d, h), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, dev(b["dy_perm"], tdt), dev(f["hp"], tdt), dw2, off,
                         M=d, N=h)
    assert rel_inf(to_np(dw2), b["dW2"]) <= tol
    dw1 = torch.full((E, 2 * h, d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_grouped_gemm(moe.MOE_GG_WGRAD, dev(b["dab"], tdt), xp, dw1, off, M=2 * h, N=d)
    assert rel_inf(to_np(dw1), b["dW1"]) <= tol
    if E >= 5:
        assert f["route"]["counts"][1] == 0
        assert torch.all(dw1[1] == 0) and torch.all(dw2[1] == 0)


# ---------------------------------------------------------------------------
# whole layer


def _run_layer(inp, k, tdt):
    w1 = dev(inp["w1"], tdt)
    w2 = dev(inp["w2"], tdt)
    layer = moe.MoELayer(w1, w2, k)
    out = layer.forward(dev(inp["x"], tdt), dev(inp["logits"], torch.float32))
    g = layer.backward(dev(inp["dout"], tdt))
    torch.cuda.synchronize()
    return layer, out, g


@pytest.mark.parametrize("shape,dt", [((256, 128, 8, 2, 256), "f32"), ((300, 256, 8, 2, 192), "bf16"),
                                      ((513, 128, 16, 4, 96), "bf16"), ((200, 64, 4, 4, 64), "f32"),
                                      # the widest d and h the library accepts (d = 16384: GEMM1's
                                      # K and GEMM2's N; h = 8192: GEMM1's N = 2h = 16384 and
                                      # GEMM2's K), and the largest E with the largest k
                                      ((64, 16384, 4, 2, 128), "bf16"), ((64, 128, 4, 2, 8192), "bf16"),
                                      ((300, 128, 256, 8, 64), "bf16"), ((300, 128, 256, 8, 64), "f32"),
                                      # h > d and d % 64 == 32
                                      ((333, 96, 7, 3, 160), "bf16"), ((200, 64, 8, 2, 512), "bf16")])
def test_layer_end_to_end(shape, dt):
    T, d, E, k, h = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp = _layer_inputs(T, d, E, k, h, seed=7, dt=dt)
    f = oracle.layer_forward(inp, k, dt)
    b = oracle.layer_backward(inp, f, k, dt)
    layer, out, g = _run_layer(inp, k, tdt)
    _route_eq(layer.route, f["route"])
    tol = TOL[dt]
    assert rel_inf(to_np(out), f["out"]) <= tol
    for key, ref in (("dx", b["dx"]), ("dw1", b["dW1"]), ("dw2", b["dW2"]),
                     ("dlogits", b["dlogits"]), ("dgate", b["dgate"])):
        assert rel_inf(to_np(g[key]), ref) <= tol, key
    # unselected experts: exactly zero logit gradient
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, f["route"]["topk_idx"].astype(np.int64), True, 1)
    assert np.all(to_np(g["dlogits"])[~sel] == 0)


def _bias(col, by):
    def f(inp):
        inp["logits"][:, col] += by
    return f


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape,mod", [
    ((1, 32, 1, 1, 32), None),                  # one token, one expert
    ((1, 64, 8, 8, 32), None),                  # one token on every expert (k = E)
    ((200, 96, 6, 2, 64), _bias(-1, -100.0)),   # the last expert gets no rows
    ((200, 64, 6, 2, 96), _bias(0, -100.0)),    # the first expert gets no rows
    # every token's first choice is expert 1 (a bias that fixes the choice
    # while the other gates, e^-10 of it, stay normal fp32 numbers)
    ((300, 128, 8, 2, 128), _bias(1, 10.0)),
])
def test_layer_edge_cases(shape, mod, dt):
    T, d, E, k, h = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp = _layer_inputs(T, d, E, k, h, seed=3, dt=dt)
    if mod:
        mod(inp)
    f = oracle.layer_forward(inp, k, dt)
    b = oracle.layer_backward(inp, f, k, dt)
    layer, out, g = _run_layer(inp, k, tdt)
    _route_eq(layer.route, f["route"])
    tol = TOL[dt]
    assert rel_inf(to_np(out), f["out"]) <= tol
    for key, ref in (("dx", b["dx"]), ("dw1", b["dW1"]), ("dw2", b["dW2"]),
                     ("dlogits", b["dlogits"]), ("dgate", b["dgate"])):
        assert rel_inf(to_np(g[key]), ref) <= tol, key


# The weight gradients' output tiles are 128 x 256 (MFMA kernels). An expert
# with more than twice the mean rows is split into 8 tile chunks, one per XCD,
# when its tile count is a multiple of 8; every other expert goes whole to one
# XCD. These shapes meet both conditions for dW2 ([d, h] = [1024, 256]: 8
# tiles) and dW1 ([2h, d] = [512, 1024]: 16 tiles).
HOT_SHAPE = (512, 1024, 8, 2, 256)


def _wgrad_split_experts(counts, T, E, k, d, h):
    thresh = 2 * -(-(T * k) // E)
    tiles = {"dW2": -(-d // 128) * -(-h // 256), "dW1": -(-(2 * h) // 128) * -(-d // 256)}
    assert all(t % 8 == 0 for t in tiles.values()), tiles
    return [e for e in range(E) if counts[e] > thresh]


def _hot(inp, case):
    # biases large enough to fix the choices, small enough that the other
    # gates (e^-10 of the hot one) keep the gradients out of the fp32
    # subnormal range
    if case == "one_hot":           # every token's first choice is expert 3
        inp["logits"][:, 3] += 10.0
    else:                           # experts 2 and 5 take every token; the others none
        inp["logits"][:, 2] += 20.0
        inp["logits"][:, 5] += 10.0


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["one_hot", "two_hot"])
def test_hot_expert_split_wgrad(case, dt):
    """Skewed routing that takes the weight gradients' hot-expert path (an
    expert split over all XCDs, beside whole experts and empty ones): the
    whole layer against the oracle, each expert's dW on its own."""
    T, d, E, k, h = HOT_SHAPE
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp = _layer_inputs(T, d, E, k, h, seed=21, dt=dt)
    _hot(inp, case)
    f = oracle.layer_forward(inp, k, dt)
    b = oracle.layer_backward(inp, f, k, dt)
    counts = f["route"]["counts"]
    hot = _wgrad_split_experts(counts, T, E, k, d, h)
    assert hot == ([3] if case == "one_hot" else [2, 5]), counts
    layer, out, g = _run_layer(inp, k, tdt)
    _route_eq(layer.route, f["route"])
    tol = TOL[dt]
    assert rel_inf(to_np(out), f["out"]) <= tol
    for key, ref in (("dx", b["dx"]), ("dlogits", b["dlogits"]), ("dgate", b["dgate"])):
        assert rel_inf(to_np(g[key]), ref) <= tol, key
    dw1, dw2 = to_np(g["dw1"]), to_np(g["dw2"])
    for e in range(E):
        if counts[e] == 0:
            assert np.all(dw1[e] == 0) and np.all(dw2[e] == 0), e
        else:
            assert rel_inf(dw1[e], b["dW1"][e]) <= tol, e
            assert rel_inf(dw2[e], b["dW2"][e]) <= tol, e


def _clobber_scratch():
    """Overwrite the shared recompute scratch, as other layers would between
    a layer's forward and its backward."""
    for t in moe._SCRATCH.values():
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(0x7F)


@pytest.mark.parametrize("shape,dt", [((300, 256, 8, 2, 192), "bf16"), ((200, 64, 4, 4, 64), "f32")])
def test_recompute_matches_saved(shape, dt):
    """recompute=True holds only y_perm and the routing metadata and rebuilds
    x_perm, A||B and H' in the backward: gradients bit-identical to the
    layer that keeps them, and within tolerance of the oracle."""
    T, d, E, k, h = shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    inp = _layer_inputs(T, d, E, k, h, seed=13, dt=dt)
    base, out0, g0 = _run_layer(inp, k, tdt)
    out0 = out0.clone()
    g0 = {key: v.clone() for key, v in g0.items() if v is not None and not key.startswith("_")}
    layer = moe.MoELayer(dev(inp["w1"], tdt), dev(inp["w2"], tdt), k, recompute=True)
    out = layer.forward(dev(inp["x"], tdt), dev(inp["logits"], torch.float32))
    torch.cuda.synchronize()
    _clobber_scratch()
    g = layer.backward(dev(inp["dout"], tdt))
    torch.cuda.synchronize()
    assert torch.equal(out, out0)
    for key in ("dx", "dw1", "dw2", "dlogits", "dgate"):
        assert torch.equal(g[key], g0[key]), key
    assert layer.held_bytes() < base.held_bytes()
    b = oracle.layer_backward(inp, oracle.layer_forward(inp, k, dt), k, dt)
    assert rel_inf(to_np(g["dx"]), b["dx"]) <= TOL[dt]
    assert rel_inf(to_np(g["dw1"]), b["dW1"]) <= TOL[dt]


def test_recompute_full_size():
    """The 16384-token E=128 workload, recomputing: bit-identical to the
    layer that keeps its activations; holds under a third of their bytes."""
    w = synth.WORKLOADS["e128_bf16"]
    d_in = synth.device_inputs(w, seed=0, with_dout=True)
    ref = moe.MoELayer(d_in["w1"], d_in["w2"], w.k)
    ref.forward(d_in["x"], d_in["logits"])
    g0 = {key: v.clone() for key, v in ref.backward(d_in["dout"]).items()
          if v is not None and key in ("dx", "dw1", "dw2", "dlogits")}
    held0 = ref.held_bytes()
    del ref
    layer = moe.MoELayer(d_in["w1"], d_in["w2"], w.k, recompute=True)
    layer.forward(d_in["x"], d_in["logits"])
    torch.cuda.synchronize()
    _clobber_scratch()
    g = layer.backward(d_in["dout"])
    torch.cuda.synchronize()
    for key, v in g0.items():
        assert torch.equal(g[key], v), key
    assert layer.held_bytes() * 3 < held0


def test_tiny_fp32_workload():
    w = synth.WORKLOADS["tiny_fp32"]
    inp = synth.host_inputs(w, 0)
    f = oracle.layer_forward(inp, w.k, "f32")
    b = oracle.layer_backward(inp, f, w.k, "f32")
    layer, out, g = _run_layer(inp, w.k, torch.float32)
    assert rel_inf(to_np(out), f["out"]) <= 1e-4
    assert rel_inf(to_np(g["dx"]), b["dx"]) <= 1e-4
    assert rel_inf(to_np(g["dw1"]), b["dW1"]) <= 1e-4


def test_deterministic():
    inp = _layer_inputs(400, 128, 8, 2, 128, seed=2)
    a = _run_layer(inp, 2, torch.bfloat16)
    o1 = a[1].clone(); g1 = {k_: v.clone() for k_, v in a[2].items() if v is not None}
    b = _run_layer(inp, 2, torch.bfloat16)
    assert torch.equal(o1, b[1])
    for key, v in g1.items():
        assert torch.equal(v, b[2][key]), key


@pytest.mark.parametrize("name", ["e128_bf16_zipf", "e128_mxfp8"])
def test_full_size_deterministic(name):
    """Two runs of the full-size layer (forward and backward, the bench's
    launch configuration) give the same bits: every output element is
    reduced by one workgroup in a fixed order, under skewed routing too."""
    w = synth.WORKLOADS[name]
    d_in = synth.device_inputs(w, seed=1, with_dout=True)
    make = (lambda: moe.MoELayerMX(d_in["w1"], d_in["w2"], w.k)) if w.dtype == "mxfp8" \
        else (lambda: moe.MoELayer(d_in["w1"], d_in["w2"], w.k))
    runs = []
    for _ in range(2):
        layer = make()
        out = layer.forward(d_in["x"], d_in["logits"]).clone()
        g = layer.backward(d_in["dout"])
        runs.append((out, {key: g[key].clone() for key in ("dx", "dw1", "dw2", "dlogits")}))
        del layer, g
        torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0])
    for key in runs[0][1]:
        assert torch.equal(runs[0][1][key], runs[1][1][key]), key


def test_zero_tokens():
    w1 = torch.randn(4, 64, 32, device="cuda").bfloat16()
    w2 = torch.randn(4, 32, 32, device="cuda").bfloat16()
    layer = moe.MoELayer(w1, w2, 2)
    out = layer.forward(torch.empty((0, 32), device="cuda", dtype=torch.bfloat16),
                        torch.empty((0, 4), device="cuda"))
    g = layer.backward(torch.empty((0, 32), device="cuda", dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert out.shape == (0, 32)
    assert torch.all(layer.route["counts"] == 0) and torch.all(layer.route["offsets"] == 0)
    assert torch.all(g["dw1"] == 0) and torch.all(g["dw2"] == 0)


# ---------------------------------------------------------------------------
# full-size workloads: sampled outputs against the oracle, in the launch
# configuration the bench times


def _sample_experts(counts, n_random, seed):
    """The hottest expert, an empty one (if any), a median-load one and
    n_random other experts with rows."""
    nz = np.flatnonzero(counts)
    hot = int(np.argmax(counts))
    med = int(nz[np.argsort(counts[nz], kind="stable")[len(nz) // 2]])
    pick = {hot, med}
    empty = np.flatnonzero(counts == 0)
    if len(empty):
        pick.add(int(empty[len(empty) // 2]))
    rest = np.array(sorted(set(nz.tolist()) - pick))
    for i in synth.sample_indices(len(rest), n_random, seed=seed):
        pick.add(int(rest[i]))
    return sorted(pick)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["e128_bf16", "e128_bf16_zipf", "e8_bf16_fwd", "e16_bf16_ep_share"])
def test_full_size_sampled(name):
    """The full-size workloads in the launch configuration the bench times:
    routing in full, 512 sampled tokens (out, dX, dlogits) and the weight
    gradients of the hottest expert, an empty one, a median one and three
    random ones against the oracle."""
    w = synth.WORKLOADS[name]
    d_in = synth.device_inputs(w, seed=0, with_dout=w.backward)
    layer = moe.MoELayer(d_in["w1"], d_in["w2"], w.k)
    out = layer.forward(d_in["x"], d_in["logits"])
    g = layer.backward(d_in["dout"]) if w.backward else None
    torch.cuda.synchronize()
    host = {key: (to_np(v) if v is not None else None) for key, v in d_in.items()}
    r = oracle.route(host["logits"], w.k)
    _route_eq(layer.route, r)
    counts = r["counts"]
    toks = synth.sample_indices(w.T, 512, seed=1)
    exps = _sample_experts(counts, 3, seed=2) if w.backward else []
    s = oracle.layer_sampled(host, w.k, "bf16", toks, exps, backward=w.backward)
    assert rel_inf(to_np(out)[toks], s["out"]) <= TOL["bf16"]
    if not w.backward:
        return
    assert rel_inf(to_np(g["dx"])[toks], s["dx"]) <= TOL["bf16"]
    assert rel_inf(to_np(g["dlogits"])[toks], s["dlogits"]) <= TOL["bf16"]
    for e in exps:
        if counts[e] == 0:
            assert torch.all(g["dw1"][e] == 0) and torch.all(g["dw2"][e] == 0), e
            continue
        assert rel_inf(to_np(g["dw1"][e]), s["dW1"][e]) <= TOL["bf16"], e
        assert rel_inf(to_np(g["dw2"][e]), s["dW2"][e]) <= TOL["bf16"], e
    for e in np.flatnonzero(counts == 0):
        assert torch.all(g["dw1"][int(e)] == 0) and torch.all(g["dw2"][int(e)] == 0)
