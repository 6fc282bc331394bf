"""The routing metadata never leaves the GPU: every call of the layer only
enqueues kernels (no allocation, no device-to-host copy, no synchronisation),
which is what lets the host run ahead of the device (Ai2 Olmo-core 3,
kongchang.com, "routing is a systems problem"; bytechap.com, "How it works").

Test: the whole forward + backward is captured once into a HIP graph (a
capture fails on any synchronisation or device-to-host copy) and replayed on
new router logits copied into the captured input. The group sizes change from
replay to replay while the host never reads them; each replay must give the
same bits as an eager layer on the same inputs, routing bit-exact against the
oracle and the outputs within the dtype's tolerance of it. Eager work and
synchronisations run between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import TOL, dev, rel_inf, to_np

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routing_grouped_gemm_router_amd as moe

ROUTE_KEYS = ("topk_idx", "counts", "offsets", "token_pos", "sorted_token", "sorted_slot")
GRAD_KEYS = ("dx", "dw1", "dw2", "dlogits", "dgate")


def _inputs(T, d, E, k, h, mx):
    inp = dict(logits=synth.normal((T, E), 31, 0, 1.0), x=synth.normal((T, d), 31, 1, 1.0),
               w1=synth.normal((E, 2 * h, d), 31, 2, 0.05 if not mx else 0.02),
               w2=synth.normal((E, d, h), 31, 3, 0.05 if not mx else 0.02),
               dout=synth.normal((T, d), 31, 4, 1.0))
    keys = ("x", "dout") if mx else ("x", "w1", "w2", "dout")
    for key in keys:
        inp[key] = torch.from_numpy(inp[key]).bfloat16().float().numpy()
    return inp


def _new_logits(T, E, i):
    lg = synth.normal((T, E), 50 + i, 0, 1.0)
    if i == 1:
        lg[:, 0] += 2.5           # a skewed round: expert 0 takes far more rows
    if i == 2:
        lg[:, E - 1] -= 100.0     # the last expert gets no rows
    return lg


@pytest.mark.parametrize("kind", ["bf16", "mxfp8"])
def test_layer_graph_replay_new_logits(kind):
    T, d, E, k, h = 512, 256, 16, 2, 128
    mx = kind == "mxfp8"
    inp = _inputs(T, d, E, k, h, mx)
    wdt = torch.float32 if mx else torch.bfloat16
    make = (lambda: moe.MoELayerMX(dev(inp["w1"], wdt), dev(inp["w2"], wdt), k)) if mx else \
        (lambda: moe.MoELayer(dev(inp["w1"], wdt), dev(inp["w2"], wdt), k))
    layer, eager = make(), make()
    x = dev(inp["x"], torch.bfloat16)
    dout = dev(inp["dout"], torch.bfloat16)
    logits = dev(inp["logits"], torch.float32)
    # warm-up on a side stream: the layer allocates its buffers here, so the
    # captured calls allocate nothing
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer.forward(x, logits)
            layer.backward(dout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = layer.forward(x, logits)
        grads = layer.backward(dout)

    seen_counts = []
    for i in range(3):
        lg = _new_logits(T, E, i)
        logits.copy_(torch.from_numpy(lg))
        graph.replay()
        torch.cuda.synchronize()
        # eager layer (its own buffers) on the same inputs, between replays
        e_out = eager.forward(x, logits).clone()
        e_g = {key: v.clone() for key, v in eager.backward(dout).items() if key in GRAD_KEYS}
        torch.cuda.synchronize()
        assert torch.equal(out, e_out), i
        for key in GRAD_KEYS:
            assert torch.equal(grads[key], e_g[key]), (i, key)
        for key in ROUTE_KEYS:
            assert torch.equal(layer.route[key], eager.route[key]), (i, key)
        # against the oracle: routing bit-exact, values within tolerance
        ref_in = dict(inp, logits=lg)
        r = oracle.route(lg, k)
        for key in ROUTE_KEYS:
            assert np.array_equal(layer.route[key].cpu().numpy(), r[key]), (i, key)
        seen_counts.append(r["counts"].copy())
        if mx:
            m = oracle.layer_mx(ref_in, k)
            ref = dict(out=m["out"], dx=m["dx"], dlogits=m["dlogits"],
                       dw1=np.stack([m["dW1"][e] for e in range(E)]),
                       dw2=np.stack([m["dW2"][e] for e in range(E)]))
        else:
            f = oracle.layer_forward(ref_in, k, "bf16")
            b = oracle.layer_backward(ref_in, f, k, "bf16")
            ref = dict(out=f["out"], dx=b["dx"], dlogits=b["dlogits"], dw1=b["dW1"], dw2=b["dW2"])
        tol = TOL[kind]
        assert rel_inf(to_np(out), ref["out"]) <= tol, i
        for key in ("dx", "dlogits", "dw1", "dw2"):
            assert rel_inf(to_np(grads[key]), ref[key]) <= tol, (i, key)
    # the group sizes changed between replays without the host reading them
    assert not np.array_equal(seen_counts[0], seen_counts[1])
    assert seen_counts[2][E - 1] == 0 and seen_counts[1][0] > seen_counts[0][0]
