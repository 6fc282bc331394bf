"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload e128_bf16]

A step is one pass of the whole path on one batch of synthetic inputs already
resident in HBM: route -> permute -> grouped GEMM1 + SwiGLU -> grouped GEMM2
-> combine, then the full backward (combine/router backward, GEMM2 dgrad +
SwiGLU backward, GEMM2 wgrad, GEMM1 dgrad, unpermute backward, GEMM1 wgrad).
Prints one JSON line. Default workload: T=16384 tokens, d=2048, E=128
experts, top-4, SwiGLU hidden 1024, bf16 with fp32 accumulation, random
routing (the pages' measurement condition: kongchang.com, "caveats behind the
numbers").

Besides the layer throughput the line carries:
  roles        -- every kernel of the step (each grouped GEMM role, the row
                  movers, routing, the MXFP8 quantisers), timed with HIP events
                  on the launch stream inside the timed region, with its
                  algorithmic flops and bytes against the MFMA and HBM peaks;
  roofline     -- the role that takes the most time per launch (the dominant
                  kernel) against the roof that binds it;
  workloads    -- the other layer configurations (E=8 forward and the
                  8 -> 128 expert per-token cost; one GPU's 16-expert share
                  of the E=128 layer under an 8-way expert split; Zipf-skewed
                  routing against the padded-capacity layout; MXFP8 against
                  bf16 on the same seed), each timed the same way after the
                  main region;
  cpu_baseline -- the CPU oracle (plain loops, fp64) on the host cores, on a
                  bounded sample: the same layer on the first few thousand
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

FWD_STAGES = {"bf16": ("route", "permute", "gemm1_swiglu", "gemm2", "combine"),
              "mxfp8": ("quant_x", "route", "permute", "gemm1_swiglu", "gemm2", "combine")}


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
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other layer configurations")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed step: skip the padded, recompute, load-balance, "
                         "accumulation, re-quantisation and other-workload sections "
                         "(for profiling runs)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens in the oracle's bounded sample")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="run a plain device copy of this many MiB (PMC byte calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work of each role (useful flops over routed rows only; the
# minimum HBM bytes: every operand read once, every output written once)


def role_work(w) -> dict:
    T, d, E, k, h, R = w.T, w.d, w.E, w.k, w.h, w.R
    mx = w.dtype == "mxfp8"
    q = 1.0 + 1.0 / 32 if mx else 2.0        # bytes per GEMM operand element (+ E8M0 scales)
    a = 2.0                                  # bf16 activations
    route = 4 * T * E + 12 * T * k + 8 * R
    W = {
        "route": (0, route),
        "permute": (0, (T + R) * d * q),
        "gemm1_swiglu": (4 * R * d * h, R * d * q + E * 2 * h * d * q + a * R * 3 * h),
        "gemm2": (2 * R * d * h, R * h * q + E * d * h * q + a * R * d),
        "combine": (0, a * R * d + 8 * T * k + a * T * d),
        "combine_bwd": (0, a * T * d + a * R * d + 12 * T * k + a * R * d + 4 * T * E + 4 * T * k),
        "gemm2_dgrad_swiglu": (2 * R * d * h, R * d * q + E * d * h * q + a * R * 4 * h),
        "gemm2_wgrad": (2 * R * d * h, R * d * q + R * h * q + 4 * E * d * h),
        "gemm1_dgrad": (4 * R * d * h, R * 2 * h * q + E * 2 * h * d * q + a * R * d),
        "unpermute_bwd": (0, a * R * d + a * T * d + 4 * T * k),
        "gemm1_wgrad": (4 * R * d * h, R * 2 * h * q + R * d * q + 8 * E * d * h),
    }
    if mx:
        # GEMM1 stores A||B in bf16 and H' quantised in both layouts (GEMM2's
        # operand and GEMM2 wgrad's), so no pass quantises H'
        W["gemm1_swiglu"] = (4 * R * d * h,
                             R * d * q + E * 2 * h * d * q + a * R * 2 * h + 2 * R * h * q)
        # the MXFP8 backward stores no dy_perm: the combine backward writes one
        # fp32 gate per routed row, and the dy quantiser reads the dOut rows
        # (each token's once at the least) and those gates
        W["combine_bwd"] = (0, a * T * d + a * R * d + 12 * T * k + 4 * R + 4 * T * E + 4 * T * k)
        W.update({
            "quant_x": (0, a * T * d + T * d * q),
            # the backward's H' quantiser has no work: the layer holds GEMM1's
            # column layout of H'
            "quant_dy_both": (0, a * T * d + 8 * R + 2 * R * d * q),     # + gates, row map
            "quant_hp_cols": (0, 0),
            "quant_dab_both": (0, a * R * 2 * h + 2 * R * 2 * h * q),
            "quant_x_cols": (0, a * R * d + R * d * q),
        })
    return W


def role_table(w, times_ms: dict) -> dict:
    """Per role: average µs per launch, TFLOP/s and GB/s of its algorithmic
    work, the fraction of each peak, and the fraction of the roof that binds
    it (max of its MFMA-limited and HBM-limited times over its time)."""
    peak = PEAK_FP8_TFLOPS if w.dtype == "mxfp8" else PEAK_BF16_TFLOPS
    work = role_work(w)
    out = {}
    for name, ms in times_ms.items():
        flops, nbytes = work.get(name, (0, 0))
        t = ms * 1e-3
        r = {"us": ms * 1e3}
        t_mfma = flops / (peak * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        if flops:
            r["tflops"] = flops / t / 1e12
            r["frac_mfma"] = r["tflops"] / peak
        if nbytes:
            r["gbps"] = nbytes / t / 1e9
            r["frac_hbm"] = r["gbps"] / PEAK_HBM_GBS
        r["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
        r["frac_roof"] = max(t_mfma, t_hbm) / t
        sp = getattr(times_ms, "spread", {}).get(name)
        if sp is not None:
            r["us_median"], r["us_min"] = sp[0] * 1e3, sp[1] * 1e3
        out[name] = r
    return out


# ---------------------------------------------------------------------------
# the timed layer step


class StageEvents:
    """HIP events for every stage of every timed step, created (recorded once)
    before the timed region so the library can record the backward ones."""

    def __init__(self, torch, stream, steps, n):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
                   for _ in range(steps)]
        for row in self.ev:
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()

    def stage_ms(self, names):
        """Average ms of stage j over the steps (event j+1 minus event j), as
        a StageTimes carrying each stage's median and minimum too, and the
        median and minimum of the whole step (first event to last)."""
        n = len(self.ev)
        out = StageTimes()
        for j, nm in enumerate(names):
            t = sorted(r[j].elapsed_time(r[j + 1]) for r in self.ev)
            out[nm] = sum(t) / n
            out.spread[nm] = (t[n // 2], t[0])
        span = sorted(r[0].elapsed_time(r[len(names)]) for r in self.ev)
        out.step = (span[n // 2], span[0])
        return out


class StageTimes(dict):
    """{stage: average ms}, with .spread = {stage: (median ms, min ms)} and
    .step = (median ms, min ms) of the step from its first to last event."""

    def __init__(self):
        super().__init__()
        self.spread = {}
        self.step = None


def make_layer(moe, w, inp):
    if w.dtype == "mxfp8":
        return moe.MoELayerMX(inp["w1"], inp["w2"], w.k)
    return moe.MoELayer(inp["w1"], inp["w2"], w.k)


def run_layer(moe, torch, w, inp, steps, warmup, layer=None, flush=None):
    """Warm-up, then `steps` timed steps (barrier + synchronize on both sides)
    with HIP events between the stages. Returns (layer, ms per step by the
    wall clock, {stage: average ms}). With `flush` (a tensor of at least
    1 GiB), every step is preceded by a write of the whole tensor, which
    evicts the 256 MB last-level cache: the stages then start cold, as a
    layer does between other layers' work (the wall-clock time then includes
    the writes and is not a step time)."""
    mx = w.dtype == "mxfp8"
    layer = layer or make_layer(moe, w, inp)
    x, logits, dout = inp["x"], inp["logits"], inp["dout"]
    T, d, k, h = w.T, w.d, w.k, w.h
    stream = torch.cuda.current_stream()
    fwd_names = FWD_STAGES["mxfp8" if mx else "bf16"]
    bwd_names = moe.BWD_STAGES["mxfp8" if mx else "bf16"] if w.backward else ()

    def step(ev):
        mark = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        mark(0)
        if mx:
            layer._alloc(T, x.device)
            layer.x = x
            moe.mxfp8_quantize(x, 1, q=layer.xq, scale=layer.xs)
            mark(1)
            r = moe.moe_route(logits, k, out=layer.route, ws=layer.route_ws)
            mark(2)
            moe.moe_permute(layer.xq, r["token_pos"], layer.xpq, x_scale=layer.xs,
                            x_perm_scale=layer.xps)
            mark(3)
            # H' leaves GEMM1 already quantised for GEMM2 and GEMM2's wgrad
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.xpq, layer.w1q, layer.ab, r["offsets"],
                                 moe.MOE_EPI_SWIGLU_FWD, N=2 * h, K=d, aux_out=layer.hpq,
                                 aux_out_scale=layer.hps, aux_out_cols=layer.hpc,
                                 aux_out_cols_scale=layer.hpcs, a_scale=layer.xps,
                                 b_scale=layer.w1s, dtype=moe.MOE_MXFP8)
            mark(4)
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.hpq, layer.w2q, layer.y_perm, r["offsets"],
                                 N=d, K=h, a_scale=layer.hps, b_scale=layer.w2s,
                                 dtype=moe.MOE_MXFP8)
            mark(5)
        else:
            layer._alloc(T, x.device, x.dtype)
            layer.x = x
            r = moe.moe_route(logits, k, out=layer.route, ws=layer.route_ws)
            mark(1)
            moe.moe_permute(x, r["token_pos"], layer.x_perm)
            mark(2)
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.x_perm, layer.w1, layer.ab, r["offsets"],
                                 moe.MOE_EPI_SWIGLU_FWD, N=2 * h, K=d, aux_out=layer.hp)
            mark(3)
            moe.moe_grouped_gemm(moe.MOE_GG_FWD, layer.hp, layer.w2, layer.y_perm, r["offsets"],
                                 N=d, K=h)
            mark(4)
        moe.moe_combine(layer.y_perm, r["topk_gate"], r["token_pos"], layer.out)
        mark(len(fwd_names))
        if w.backward:
            layer.backward(dout, stage_events=ev[len(fwd_names) + 1:] if ev is not None else None)

    for i in range(warmup):
        if flush is not None:
            flush.fill_(float(i))
        step(None)
    evs = StageEvents(torch, stream, steps, len(fwd_names) + len(bwd_names))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))
        step(evs.ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return layer, elapsed * 1e3 / steps, evs.stage_ms(list(fwd_names) + list(bwd_names))


def dominant_roofline(w, roles: dict, traffic) -> dict:
    """The grouped-GEMM role with the longest launch, against its binding roof."""
    gemms = {n: r for n, r in roles.items() if n.startswith("gemm")}
    name = max(gemms, key=lambda n: gemms[n]["us"])
    r = gemms[name]
    flops, nbytes = role_work(w)[name]
    mx = w.dtype == "mxfp8"
    mode = "WGRAD" if "wgrad" in name else ("DGRAD" if "dgrad" in name else "FWD")
    # every role runs on the split-role kernel except the SwiGLU backward
    kname = "gg_mfma" if name == "gemm2_dgrad_swiglu" else "gg_ws"
    kern = f"{kname}<{mode}, {'MXFP8' if mx else 'bf16'}> ({name})"
    out = {"kernel": kern, "bound": r["bound"], "traffic": traffic,
           "avg_launch_ms": r["us"] * 1e-3, "flops_per_launch": flops, "bytes_per_launch": nbytes}
    if r["bound"] == "hbm":
        out.update(achieved=r["gbps"], peak=PEAK_HBM_GBS, unit="GB/s", frac=r["frac_hbm"])
    else:
        peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
        out.update(achieved=r["tflops"], peak=peak, unit="TFLOP/s", frac=r["frac_mfma"])
    out["frac_mfma"] = r.get("frac_mfma")
    return out


def workload_summary(w, ms, stages):
    flops = w.fwd_bwd_flops() if w.backward else w.fwd_flops()
    peak = PEAK_FP8_TFLOPS if w.dtype == "mxfp8" else PEAK_BF16_TFLOPS
    roles = role_table(w, stages)
    return {"ms_per_step": ms, "tokens_per_s": w.T / (ms * 1e-3),
            "layer_tflops": flops / (ms * 1e-3) / 1e12,
            "layer_frac_of_mfma_peak": flops / (ms * 1e-3) / 1e12 / peak,
            "fwd_us": sum(stages[n] for n in FWD_STAGES["mxfp8" if w.dtype == "mxfp8" else "bf16"])
            * 1e3,
            "roles": roles}


def describe(w):
    return (f"{w.name}: MoE expert layer {'fwd+bwd' if w.backward else 'fwd'}, "
            f"T={w.T} tokens, d_model={w.d}, E={w.E} experts, top-{w.k}, SwiGLU hidden={w.h}, "
            + ("MXFP8 GEMMs and dispatch (E4M3 + E8M0/32), bf16 activations, fp32 accumulate"
               if w.dtype == "mxfp8" else "bf16 storage / fp32 accumulate")
            + f", {'Zipf(1.2)-skewed' if w.zipf_s else 'uniform random'} routing")


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
    mx = w.dtype == "mxfp8"
    print(f"[bench] {w.name}: warm-up {a.warmup}, timed {a.steps}", file=sys.stderr, flush=True)
    layer, ms, stages = run_layer(moe, torch, w, inp, a.steps, a.warmup)
    summ = workload_summary(w, ms, stages)
    print(f"[bench] {w.name}: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # HBM bytes per launch of the dominant kernel from the committed counter
    # summary, only while the GEMM sources are the ones it was measured on
    from routing_grouped_gemm_router_amd import rocprof_summary as rps
    dom = max((n for n in summ["roles"] if n.startswith("gemm")), key=lambda n: summ["roles"][n]["us"])
    tr = rps.read_traffic(os.path.join(ROOT, "profiles", f"{dom}_{w.name}_pmc.md"))
    traffic = tr[0] if tr is not None and tr[1] == rps.gemm_source_hash() else None

    res = {
        "metric": METRIC,
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "step_ms_median": stages.step[0] if getattr(stages, "step", None) else None,
        "step_ms_min": stages.step[1] if getattr(stages, "step", None) else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w), "tokens": w.T, "d_model": w.d, "experts": w.E,
                   "top_k": w.k, "hidden": w.h, "layer_tflops": summ["layer_tflops"],
                   "layer_frac_of_mfma_peak": summ["layer_frac_of_mfma_peak"]},
        "roofline": dominant_roofline(w, summ["roles"], traffic),
        "roles": summ["roles"],
    }

    if a.no_extras:
        a.no_padded = a.no_recompute = a.no_workloads = True
    extras = not a.no_extras
    if not mx and w.backward and not a.no_padded:
        res["padded_baseline"] = padded_baseline(moe, torch, inp, w, a.steps, a.warmup, ms)
    if w.backward and not a.no_recompute:
        rc = recompute_variant(moe, torch, inp, w, a.steps, a.warmup)
        rc["held_bytes_saving_layer"] = layer.held_bytes()
        rc["held_frac"] = rc["held_bytes"] / layer.held_bytes()
        rc["throughput_frac"] = ms / rc["ms_per_step"]
        res["recompute"] = rc
    if extras:
        # every stage again, each step preceded by a 1 GiB write that evicts
        # the last-level cache: what the row movers reach on cold data
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        _, _, st_cold = run_layer(moe, torch, w, inp, min(a.steps, 10), 2, layer=layer, flush=flush)
        del flush
        res["roles_flushed"] = role_table(w, st_cold)
        res["sclk"] = sample_sclk(torch, lambda: run_layer(moe, torch, w, inp, 1, 0, layer=layer))
        res["load_balance"] = load_balance_report(moe, torch, inp, layer, w)
        if w.backward:
            res["grad_accumulation"] = grad_accumulation(moe, torch, layer, inp, w, a.steps, ms)
        if mx:
            res["weight_requant"] = weight_requant(moe, torch, inp, layer, w)
    if a.copy_calib:
        n = a.copy_calib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not a.no_workloads and w.name == "e128_bf16":
        fwd_us_e128 = summ["fwd_us"]
        del layer
        inp = None
        torch.cuda.empty_cache()
        res["workloads"] = other_workloads(moe, torch, synth, a, fwd_us_e128, ms)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(synth.device_inputs(w, seed=a.seed, with_dout=w.backward)
                                           if inp is None else inp, w, a.cpu_tokens)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
# the other configurations, timed like the main step after the main region


def other_workloads(moe, torch, synth, a, fwd_us_e128, ms_e128):
    out = {}
    # E=8 forward: the same d, h and k as the headline with 8 instead of 128
    # experts (the pages' expert-pool scaling: 8 -> 128 experts at top-4 cost
    # little throughput; kongchang.com, "expert-pool scaling")
    w8 = synth.WORKLOADS["e8_bf16_fwd"]
    inp = synth.device_inputs(w8, seed=a.seed, with_dout=False)
    print(f"[bench] {w8.name}", file=sys.stderr, flush=True)
    _, ms, st = run_layer(moe, torch, w8, inp, a.steps, a.warmup)
    out[w8.name] = workload_summary(w8, ms, st)
    e8 = out[w8.name]["fwd_us"] / w8.T
    e128 = fwd_us_e128 / synth.WORKLOADS["e128_bf16"].T
    out["expert_scaling"] = {"fwd_us_per_token_e8": e8, "fwd_us_per_token_e128": e128,
                             "e128_throughput_over_e8": e8 / e128}
    del inp
    torch.cuda.empty_cache()

    # one GPU's share of the E=128 layer under an 8-way expert split: 16
    # experts x ~512 rows, the per-GPU grouped GEMM work of that layout (the
    # row exchange between GPUs is not part of a one-GPU run)
    we = synth.WORKLOADS["e16_bf16_ep_share"]
    inp = synth.device_inputs(we, seed=a.seed)
    print(f"[bench] {we.name}", file=sys.stderr, flush=True)
    _, ms, st = run_layer(moe, torch, we, inp, a.steps, a.warmup)
    out[we.name] = workload_summary(we, ms, st)
    out[we.name]["us_per_token_over_e128"] = (ms / we.T) / (ms_e128 / synth.WORKLOADS["e128_bf16"].T)
    del inp
    torch.cuda.empty_cache()

    # Zipf-skewed routing, dropless against every expert padded to capacity
    # 1.25 (kongchang.com, "routing is a systems problem")
    wz = synth.WORKLOADS["e128_bf16_zipf"]
    inp = synth.device_inputs(wz, seed=a.seed)
    print(f"[bench] {wz.name}", file=sys.stderr, flush=True)
    layer, ms, st = run_layer(moe, torch, wz, inp, a.steps, a.warmup)
    out[wz.name] = workload_summary(wz, ms, st)
    counts = layer.route["counts"].cpu()
    out[wz.name]["max_rows_over_mean"] = float(counts.max()) * wz.E / wz.R
    out[wz.name]["empty_experts"] = int((counts == 0).sum())
    del layer
    torch.cuda.empty_cache()
    out[wz.name]["padded_baseline"] = padded_baseline(moe, torch, inp, wz, a.steps, a.warmup, ms)
    torch.cuda.empty_cache()
    # padding without drops needs every expert at the largest load
    cmax = int(counts.max())
    out[wz.name]["padded_no_drop"] = padded_baseline(moe, torch, inp, wz, max(2, a.steps // 4), 1,
                                                     ms, capacity=cmax)
    del inp
    torch.cuda.empty_cache()

    # MXFP8 against bf16 on the same seed (the pages' MXFP8 vs BF16 comparison,
    # kongchang.com "caveats behind the numbers"; aikraft.ru, technical
    # optimisations): fp32 masters quantised to MXFP8 for one layer, rounded to
    # bf16 for the other; same logits, x and dOut
    wm = synth.WORKLOADS["e128_mxfp8"]
    inp = synth.device_inputs(wm, seed=a.seed)
    print(f"[bench] {wm.name}", file=sys.stderr, flush=True)
    lmx, ms_mx, st = run_layer(moe, torch, wm, inp, a.steps, a.warmup)
    out[wm.name] = workload_summary(wm, ms_mx, st)
    out_mx = lmx.out.float()
    dx_mx = lmx.grads["dx"].float()
    del lmx
    torch.cuda.empty_cache()
    inp_b = dict(inp, w1=inp["w1"].bfloat16(), w2=inp["w2"].bfloat16())
    del inp
    wb = synth.Workload("e128_mxfp8_shape_bf16", wm.T, wm.d, wm.E, wm.k, wm.h, "bf16",
                        wm.logit_scale, wm.x_scale, wm.w_scale)
    print(f"[bench] {wb.name}", file=sys.stderr, flush=True)
    lb, ms_b, st = run_layer(moe, torch, wb, inp_b, a.steps, a.warmup)
    sb = workload_summary(wb, ms_b, st)

    def rel(x, ref):
        return {"inf": float((x - ref).abs().max() / ref.abs().max()),
                "fro": float((x - ref).norm() / ref.norm())}

    out[wm.name]["bf16_same_seed"] = {
        "ms_per_step": ms_b, "tokens_per_s": sb["tokens_per_s"],
        "layer_frac_of_mfma_peak": sb["layer_frac_of_mfma_peak"], "roles": sb["roles"],
        "mxfp8_speedup": ms_b / ms_mx,
        "rel_diff_out": rel(out_mx, lb.out.float()),
        "rel_diff_dx": rel(dx_mx, lb.grads["dx"].float()),
    }
    del lb, inp_b
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# variants of the headline layer


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


def grad_accumulation(moe, torch, layer, inp, w, steps, ms_overwrite):
    """A micro-batch step whose backward adds dW1, dW2 into the previous
    micro-batch's (accumulate_dw), against the main step that overwrites
    them; outside the main timed region."""
    x, logits, dout = inp["x"], inp["logits"], inp["dout"]
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


def padded_baseline(moe, torch, inp, w, steps, warmup, ms_dropless, capacity=None):
    """The padded-capacity alternative on the same inputs: the same kernels,
    every expert padded to `capacity` rows (default ceil(1.25 T*k / E)),
    overflow rows dropped. Timed like the main loop, after it (outside the
    main timed region)."""
    import synth

    C = synth.capacity(w) if capacity is None else capacity
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
    ms = el * 1e3 / steps
    return {"capacity": C, "computed_rows": w.E * C, "routed_rows": w.R,
            "dropped_frac": dropped / w.R, "ms_per_step": ms,
            "tokens_per_s": w.T * steps / el, "dropless_speedup": ms / ms_dropless}


def sample_sclk(torch, run_step, seconds: float = 0.6):
    """The GPU's graphics clock (MHz) and socket power (W) sampled every 10 ms
    while the step runs back to back, from amd-smi; the GPU with the most
    graphics activity meanwhile is the one reported, with its power cap (the
    row GEMMs run at it, which is what holds the clock below 2.4 GHz). None
    if amd-smi is not usable."""
    try:
        import threading
        import amdsmi
    except ImportError:
        return None
    try:
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        clk = {i: [] for i in range(len(handles))}
        act = {i: [] for i in range(len(handles))}
        pwr = {i: [] for i in range(len(handles))}
        stop = threading.Event()

        def poll():
            while not stop.is_set():
                for i, hdl in enumerate(handles):
                    try:
                        c = amdsmi.amdsmi_get_clock_info(hdl, amdsmi.AmdSmiClkType.GFX)["clk"]
                        a = amdsmi.amdsmi_get_gpu_activity(hdl)["gfx_activity"]
                    except Exception:
                        continue
                    try:
                        p = amdsmi.amdsmi_get_power_info(hdl).get("current_socket_power")
                    except Exception:
                        p = None
                    clk[i].append(c)
                    act[i].append(a)
                    pwr[i].append(p)
                time.sleep(0.01)

        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t0 = time.time()
        while time.time() - t0 < seconds:
            run_step()
            torch.cuda.synchronize()
        stop.set()
        th.join(timeout=5)
        busy = [i for i in clk if clk[i] and act[i]]
        if not busy:
            return None
        i = max(busy, key=lambda j: sum(act[j]) / len(act[j]))
        # the samples taken while the graphics engine was busy (at least half
        # the highest activity read), so that gaps between steps do not count
        num = (int, float)
        trip = [(c, a, p) for c, a, p in zip(clk[i], act[i], pwr[i])
                if isinstance(c, num) and isinstance(a, num)]
        top = max((a for _, a, _ in trip), default=0)
        busy_s = [(c, p) for c, a, p in trip if top > 0 and a >= top / 2]
        c = sorted(c for c, _ in busy_s)
        if not c:
            return None
        res = {"median_mhz": c[len(c) // 2], "min_mhz": c[0], "max_mhz": c[-1], "samples": len(c),
               "all_samples": len(trip), "spec_mhz": 2400}
        p = sorted(p for _, p in busy_s if isinstance(p, num))
        if p:
            res.update(power_median_w=p[len(p) // 2], power_max_w=p[-1])
            try:
                cap = amdsmi.amdsmi_get_power_cap_info(handles[i])["power_cap"]
                res["power_cap_w"] = cap / 1e6 if cap > 1e5 else cap   # reported in uW
            except Exception:
                pass
        return res
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, w, n_tok):
    """The oracle, untuned, on the host cores: the same layer (all E experts,
    same weights) forward + backward on the workload's first n_tok tokens,
    with the wall time of each of its stages."""
    import oracle

    sub = dict(logits=inp["logits"][:n_tok].float().cpu().numpy(),
               x=inp["x"][:n_tok].float().cpu().numpy(),
               w1=inp["w1"].float().cpu().numpy(), w2=inp["w2"].float().cpu().numpy(),
               dout=inp["dout"][:n_tok].float().cpu().numpy() if w.backward else None)
    stages = {}
    t0 = time.perf_counter()
    if w.dtype == "mxfp8":
        oracle.layer_mx(sub, w.k, backward=w.backward)
    else:
        f = oracle.layer_forward(sub, w.k, "bf16", timings=stages)
        if w.backward:
            oracle.layer_backward(sub, f, w.k, "bf16", timings=stages)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {n_tok} of {w.T} tokens of {w.name} (all {w.E} experts), "
                      f"{'fwd+bwd' if w.backward else 'fwd'}, fp64 oracle, {dt:.1f} s",
            "cpu_model": cpu_model(), "stage_s": stages, "single_thread": cpu_single_thread()}


def cpu_single_thread() -> dict:
    """The oracle on one host thread: the whole tiny_fp32 workload (fwd+bwd)
    and the first 32 tokens of e8_bf16_fwd (its forward), in tokens/s."""
    import oracle
    import synth

    n0 = oracle.threads()
    out = {}
    try:
        oracle.set_threads(1)
        for name, n_tok in (("tiny_fp32", None), ("e8_bf16_fwd", 32)):
            w = synth.WORKLOADS[name]
            h = synth.host_inputs(w, seed=0, with_dout=w.backward)
            n = w.T if n_tok is None else n_tok
            sub = dict(logits=h["logits"][:n], x=h["x"][:n], w1=h["w1"], w2=h["w2"],
                       dout=h["dout"][:n] if w.backward else None)
            dt = "f32" if w.dtype == "f32" else "bf16"
            t0 = time.perf_counter()
            f = oracle.layer_forward(sub, w.k, dt)
            if w.backward:
                oracle.layer_backward(sub, f, w.k, dt)
            el = time.perf_counter() - t0
            out[name] = {"tokens": n, "pass": "fwd+bwd" if w.backward else "fwd",
                         "seconds": el, "tokens_per_s": n / el}
    finally:
        oracle.set_threads(n0)
    return out


if __name__ == "__main__":
    main()
