"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload e128_bf16]

A step is one pass of the whole path on one batch of synthetic inputs already
resident in HBM: route -> permute -> grouped GEMM1 + SwiGLU -> grouped GEMM2
-> combine, then the full backward (combine/router backward, GEMM2 dgrad +
SwiGLU backward, GEMM2 wgrad, GEMM1 dgrad, GEMM1 wgrad, unpermute backward).
Prints one JSON line. Default workload: T=16384 tokens, d=2048, E=128
experts, top-4, SwiGLU hidden 1024, bf16 with fp32 accumulation, random
routing (the pages' measurement condition: kongchang.com, "caveats behind the
numbers").

Besides the layer throughput the line carries:
  roofline     -- the grouped GEMM1 + SwiGLU kernel (the largest forward
                  GEMM): useful flops 2*R*d*2h per launch over its average
                  duration, timed with HIP events on the launch stream inside
                  the timed region, against the dense bf16 MFMA peak;
  cpu_baseline -- the CPU oracle (plain loops, fp64) on the host cores, on a
                  bounded sample: the same layer on the first few hundred
                  tokens of the workload (all experts), in tokens/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s, E=128 top-4; grouped-GEMM % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="e128_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true",
                    help="skip the padded-capacity comparison (bf16 fwd+bwd workloads)")
    ap.add_argument("--no-recompute", action="store_true",
                    help="skip the recompute variant (GEMM1 rerun in the backward)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed step: skip the padded, recompute, load-balance, "
                         "accumulation and re-quantisation sections (for profiling runs)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens in the oracle's bounded sample")
    ap.add_argument("--breakdown", action="store_true",
                    help="also time every ABI call separately (stderr)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="run a plain device copy of this many MiB (PMC byte calibration)")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the MoE layer here is "
              "a single-GPU build with no collectives", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import routing_grouped_gemm_router_amd as moe

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = synth.WORKLOADS[a.workload]
    if w.dtype not in ("bf16", "mxfp8"):
        print(f"workload {w.name} is not a bf16 or MXFP8 workload", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    inp = synth.device_inputs(w, seed=a.seed, with_dout=w.backward)
    T, d, E, k, h = w.T, w.d, w.E, w.k, w.h
    R = T * k
    mx = w.dtype == "mxfp8"
    # MXFP8: the fp32 masters are quantised (both orientations) once per weight
    # update, outside the step, as a training step would between optimizer steps
    layer = moe.MoELayerMX(inp["w1"], inp["w2"], k) if mx else moe.MoELayer(inp["w1"], inp["w2"], k)
    x, logits, dout = inp["x"], inp["logits"], inp["dout"]
    stream = torch.cuda.current_stream()

    ev = []

    def gemm1(r):
        if mx:
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.xpq, layer.w1q, layer.ab, r["offsets"],
                                 moe.MOE_EPI_SWIGLU_FWD, N=2 * h, K=d, aux_out=layer.hp,
                                 a_scale=layer.xps, b_scale=layer.w1s, dtype=moe.MOE_MXFP8)
        else:
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.x_perm, layer.w1, layer.ab, r["offsets"],
                                 moe.MOE_EPI_SWIGLU_FWD, N=2 * h, K=d, aux_out=layer.hp)

    def step(timed):
        if mx:
            layer._alloc(T, x.device)
            layer.x = x
            moe.mxfp8_quantize(x, 1, q=layer.xq, scale=layer.xs)
            r = moe.moe_route(logits, k, out=layer.route, ws=layer.route_ws)
            moe.moe_permute(layer.xq, r["token_pos"], layer.xpq, x_scale=layer.xs,
                            x_perm_scale=layer.xps)
        else:
            layer._alloc(T, x.device, x.dtype)
            r = moe.moe_route(logits, k, out=layer.route, ws=layer.route_ws)
            moe.moe_permute(x, r["token_pos"], layer.x_perm)
        if timed:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        gemm1(r)
        if timed:
            e1.record(stream)
            ev.append((e0, e1))
        if mx:
            moe.mxfp8_quantize(layer.hp, 1, q=layer.hpq, scale=layer.hps)
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.hpq, layer.w2q, layer.y_perm, r["offsets"],
                                 N=d, K=h, a_scale=layer.hps, b_scale=layer.w2s,
                                 dtype=moe.MOE_MXFP8)
        else:
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.hp, layer.w2, layer.y_perm, r["offsets"],
                                 N=d, K=h)
        moe.moe_combine(layer.y_perm, r["topk_gate"], r["token_pos"], layer.out)
        if w.backward:
            layer.backward(dout)

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms = elapsed * 1e3 / a.steps
    g1_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    g1_flops = 2.0 * R * d * 2 * h
    g1_tflops = g1_flops / (g1_ms * 1e-3) / 1e12
    flops = w.fwd_bwd_flops() if w.backward else w.fwd_flops()
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS

    if a.no_extras:
        a.no_padded = a.no_recompute = True
    padded = None
    if not mx and w.backward and not a.no_padded:
        padded = padded_baseline(moe, torch, inp, w, a.steps, a.warmup)
        padded["dropless_speedup"] = padded["ms_per_step"] / ms
    extras = not a.no_extras
    balance = load_balance_report(moe, torch, inp, layer, w) if extras else None
    accum = grad_accumulation(moe, torch, layer, x, logits, dout, w, a.steps, ms) \
        if w.backward and extras else None
    requant = weight_requant(moe, torch, inp, layer, w) if mx and extras else None
    recompute = None
    if w.backward and not a.no_recompute:
        recompute = recompute_variant(moe, torch, inp, w, a.steps, a.warmup)
        recompute["held_bytes_saving_layer"] = layer.held_bytes()
        recompute["held_frac"] = recompute["held_bytes"] / layer.held_bytes()
        recompute["throughput_frac"] = ms / recompute["ms_per_step"]
    if a.breakdown and not mx:
        breakdown(moe, torch, layer, x, logits, dout, w)
    if a.copy_calib:
        n = a.copy_calib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # HBM bytes per launch of this kernel from the committed counter summary,
    # only while the kernel's sources are the ones it was measured on
    from routing_grouped_gemm_router_amd import rocprof_summary as rps
    tr = rps.read_traffic(os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                       f"gemm1_swiglu_{w.name}_pmc.md"))
    traffic = tr[0] if tr is not None and tr[1] == rps.gemm_source_hash() else None

    res = {
        "metric": METRIC,
        "value": T * a.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: MoE expert layer {'fwd+bwd' if w.backward else 'fwd'}, "
                        f"T={T} tokens, d_model={d}, E={E} experts, top-{k}, SwiGLU hidden={h}, "
                        + ("MXFP8 GEMMs and dispatch (E4M3 + E8M0/32), bf16 activations, "
                           "fp32 accumulate" if mx else "bf16 storage / fp32 accumulate")
                        + f", {'Zipf(1.2)-skewed' if w.zipf_s else 'uniform random'} routing",
            "tokens": T, "d_model": d, "experts": E, "top_k": k, "hidden": h,
            "layer_tflops": flops / (ms * 1e-3) / 1e12,
            "layer_frac_of_mfma_peak": flops / (ms * 1e-3) / 1e12 / peak,
        },
        "roofline": {
            "kernel": f"grouped GEMM1 + SwiGLU forward (gg_mfma<FWD, SWIGLU_FWD, {'MXFP8' if mx else 'bf16'}>)",
            "bound": "mfma",
            "achieved": g1_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": g1_tflops / peak,
            "traffic": traffic,
            "avg_launch_ms": g1_ms,
            "flops_per_launch": g1_flops,
        },
    }
    if padded is not None:
        res["padded_baseline"] = padded
    if recompute is not None:
        res["recompute"] = recompute
    if balance is not None:
        res["load_balance"] = balance
    if accum is not None:
        res["grad_accumulation"] = accum
    if requant is not None:
        res["weight_requant"] = requant
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, w, a.cpu_tokens)
    print(json.dumps(res), flush=True)


def load_balance_report(moe, torch, inp, layer, w, reps=20, alpha=0.01):
    """The balancing loss and load statistics of the workload's routing
    (moe_load_balance on the layer's last routing), and the call's time with
    and without the gradient pass; outside the timed step."""
    logits, counts = inp["logits"], layer.route["counts"]
    dl = torch.zeros_like(logits)
    st = moe.moe_load_balance(logits, counts, w.k, alpha)
    times = {}
    for name, grad in (("us_stats", None), ("us_stats_and_grad", dl)):
        moe.moe_load_balance(logits, counts, w.k, alpha, dlogits=grad)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            moe.moe_load_balance(logits, counts, w.k, alpha, dlogits=grad)
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) * 1e3 / reps
    vals = st.cpu().tolist()
    out = {"alpha": alpha, **{n: v for n, v in zip(moe.LB_STAT_NAMES, vals)}}
    out.update(times)
    return out


def grad_accumulation(moe, torch, layer, x, logits, dout, w, steps, ms_overwrite):
    """A micro-batch step whose backward adds dW1, dW2 into the previous
    micro-batch's (accumulate_dw), against the main step that overwrites
    them; outside the main timed region."""
    layer.forward(x, logits)
    layer.backward(dout)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, logits)
        layer.backward(dout, accumulate_dw=True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return {"ms_per_step": el * 1e3 / steps, "tokens_per_s": w.T * steps / el,
            "extra_ms_vs_overwrite": el * 1e3 / steps - ms_overwrite,
            "dw_bytes": 4 * w.E * 3 * w.d * w.h}


def weight_requant(moe, torch, inp, layer, w, reps=5):
    """Once-per-optimizer-step re-quantisation of the fp32 master weights to
    MXFP8 in both orientations: fused (each master read once) against four
    separate mxfp8_quantize calls (each master read twice)."""
    E, d, h = w.E, w.d, w.h
    w1, w2 = inp["w1"], inp["w2"]
    g1 = torch.arange(0, E + 1, dtype=torch.int32, device="cuda") * (2 * h)
    g2 = torch.arange(0, E + 1, dtype=torch.int32, device="cuda") * d

    def separate():
        moe.mxfp8_quantize(w1.reshape(E * 2 * h, d), 1)
        moe.mxfp8_quantize(w2.reshape(E * d, h), 1)
        moe.mxfp8_quantize(w1.reshape(E * 2 * h, d), 0, g1)
        moe.mxfp8_quantize(w2.reshape(E * d, h), 0, g2)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    fused_ms = timed(lambda: layer.prepare_weights(w1, w2))
    sep_ms = timed(separate)
    n = E * 3 * d * h                                    # master elements
    algo = n * 4 + 2 * (n + n // 32)                     # read once, write both orientations
    return {"fused_ms": fused_ms, "separate_ms": sep_ms, "algorithmic_bytes": algo,
            "fused_GBps": algo / (fused_ms * 1e-3) / 1e9}


def recompute_variant(moe, torch, inp, w, steps, warmup):
    """The layer that holds only y_perm and the routing metadata between its
    forward and backward and reruns dispatch + GEMM1 in the backward, on the
    same inputs; timed like the main loop, after it."""
    mx = w.dtype == "mxfp8"
    cls = moe.MoELayerMX if mx else moe.MoELayer
    layer = cls(inp["w1"], inp["w2"], w.k, recompute=True)

    def step():
        layer.forward(inp["x"], inp["logits"])
        layer.backward(inp["dout"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return {"ms_per_step": el * 1e3 / steps, "tokens_per_s": w.T * steps / el,
            "held_bytes": layer.held_bytes()}


def padded_baseline(moe, torch, inp, w, steps, warmup):
    """The padded-capacity alternative on the same inputs: the same kernels,
    every expert padded to ceil(1.25 T*k / E) rows, overflow rows dropped.
    Timed like the main loop, after it (outside the main timed region)."""
    import synth

    C = synth.capacity(w)
    layer = moe.MoELayerPadded(inp["w1"], inp["w2"], w.k, C)

    def step():
        layer.forward(inp["x"], inp["logits"])
        layer.backward(inp["dout"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    dropped = int((layer.pad["token_pos"] < 0).sum().item())
    return {"capacity": C, "computed_rows": w.E * C, "routed_rows": w.R,
            "dropped_frac": dropped / w.R, "ms_per_step": el * 1e3 / steps,
            "tokens_per_s": w.T * steps / el}


def cpu_baseline(inp, w, n_tok):
    """The oracle, untuned, on the host cores: the same layer (all E experts,
    same weights) forward + backward on the workload's first n_tok tokens."""
    import numpy as np
    import oracle

    sub = dict(logits=inp["logits"][:n_tok].float().cpu().numpy(),
               x=inp["x"][:n_tok].float().cpu().numpy(),
               w1=inp["w1"].float().cpu().numpy(), w2=inp["w2"].float().cpu().numpy(),
               dout=inp["dout"][:n_tok].float().cpu().numpy() if w.backward else None)
    t0 = time.perf_counter()
    if w.dtype == "mxfp8":
        oracle.layer_mx(sub, w.k, backward=w.backward)
    else:
        f = oracle.layer_forward(sub, w.k, "bf16")
        if w.backward:
            oracle.layer_backward(sub, f, w.k, "bf16")
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {n_tok} of {w.T} tokens of {w.name} (all {w.E} experts), "
                      f"{'fwd+bwd' if w.backward else 'fwd'}, fp64 oracle, {dt:.1f} s"}


def breakdown(moe, torch, layer, x, logits, dout, w, reps=5):
    """Per-call event timing of one step (a separate, untimed pass)."""
    T, d, E, k, h = w.T, w.d, w.E, w.k, w.h
    R = T * k
    r = layer.route
    calls = [
        ("route", lambda: moe.moe_route(logits, k, out=r, ws=layer.route_ws), 0, 4 * T * E),
        ("permute", lambda: moe.moe_permute(x, r["token_pos"], layer.x_perm), 0, 2 * T * d * (1 + k)),
        ("gemm1_swiglu", lambda: moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.x_perm, layer.w1, layer.ab,
                                                      r["offsets"], moe.MOE_EPI_SWIGLU_FWD, N=2 * h,
                                                      K=d, aux_out=layer.hp), 4 * R * d * h, 0),
        ("gemm2", lambda: moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.hp, layer.w2, layer.y_perm,
                                               r["offsets"], N=d, K=h), 2 * R * d * h, 0),
        ("combine", lambda: moe.moe_combine(layer.y_perm, r["topk_gate"], r["token_pos"], layer.out),
         0, 2 * T * d * (1 + k)),
        ("backward(all)", lambda: layer.backward(dout), 12 * R * d * h, 0),
    ]
    for name, fn, flops, nbytes in calls:
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        extra = ""
        if flops:
            extra += f" {flops / ms / 1e9:.1f} TFLOP/s ({flops / ms / 1e9 / PEAK_BF16_TFLOPS:.1%})"
        if nbytes:
            extra += f" {nbytes / ms / 1e6:.0f} GB/s ({nbytes / ms / 1e6 / PEAK_HBM_GBS:.1%})"
        print(f"[breakdown] {name:14s} {ms * 1e3:9.1f} us{extra}", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
