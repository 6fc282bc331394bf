"""Planted mistakes: each copy of the oracle with one plausible slip (a
swapped operand, a dropped term, a wrong sign or index, a wrong rounding) must
fail at least one of the pins. Mistakes are planted in a private copy of the
oracle source, compiled on the CPU; the real oracle is untouched."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")
GOLD = os.path.join(os.path.dirname(__file__), "golden")

MUTATIONS = {
    "swiglu_swapped": ("hp[j] = round_to(c->dt, silu(a) * b);", "hp[j] = round_to(c->dt, silu(b) * a);"),
    "tie_to_higher_index": ("if (best < 0 || l[e] > l[best]) best = e;",
                            "if (best < 0 || l[e] >= l[best]) best = e;"),
    "router_bwd_sign": ("(float)(g * (dgate[t * k + j] - dot))", "(float)(g * (dot - dgate[t * k + j]))"),
    "slot_index": ("sorted_slot[p] = j;", "sorted_slot[p] = k - 1 - j;"),
    "dB_uses_b": ("dab[h + j] = round_to(c->dt, g[j] * a * s);", "dab[h + j] = round_to(c->dt, g[j] * b * s);"),
    "dA_dropped_term": ("g[j] * b * s * (1.0 + a * (1.0 - s))", "g[j] * b * s"),
    "combine_bwd_no_gate": ("dy_perm[p * d + q] = round_to(dt, g * dout[t * d + q]);",
                            "dy_perm[p * d + q] = round_to(dt, dout[t * d + q]);"),
    "gemm2_reads_unrounded": ("const double *g2 = c->hp_in ? c->hp_in + r * h : hp;",
                              "const double *g2 = c->hp_in ? c->hp_in + r * h : hp; (void)g2; double hpu[4096]; for (int j2 = 0; j2 < h; j2++) hpu[j2] = silu(ab[j2]) * ab[h + j2]; g2 = hpu;"),
    "e4m3_floor": ("double r = ldexp(nearbyint(ldexp(a, 3 - E)), E - 3);",
                   "double r = ldexp(floor(ldexp(a, 3 - E)), E - 3);"),
    "mx_scale_emax7": ("int s = (e - 1) - 8;", "int s = (e - 1) - 7;"),
    "bf16_truncate": ("double q = nearbyint(ldexp(x, 8 - e));", "double q = trunc(ldexp(x, 8 - e));"),
    "combine_slot_order": ("s += (double)gate[t * k + j] * y_perm[(int64_t)token_pos[t * k + j] * d + q];",
                           "s += (double)gate[t * k + j] * y_perm[(int64_t)token_pos[t * k + (k - 1 - j)] * d + q];"),
    "wgrad_not_rounded_f32": ("for (int j = 0; j < c->nn; j++) out[j] = (double)(float)out[j];",
                              "for (int j = 0; j < c->nn; j++) out[j] = out[j] * (1.0 + 1e-3);"),
    "unpermute_drops_last_slot": ("for (int j = 0; j < k; j++) s += dx_perm[",
                                  "for (int j = 0; j < k - 1; j++) s += dx_perm["),
    "mx_rows_amax_skips_first": ("for (int i = 0; i < 32; i++) if (fabs((double)v[i]) > amax)",
                                 "for (int i = 1; i < 32; i++) if (fabs((double)v[i]) > amax)"),
    "mx_cols_amax_drops_last": ("for (int64_t i = i0; i < i1; i++) {\n            double v = fabs(",
                                "for (int64_t i = i0; i < i1 - 1; i++) {\n            double v = fabs("),
    "mx_cols_padding_nonzero": ("                : 0;\n", "                : 1;\n"),
    "mx_groups_padded_to_64": (
        "nb = 4 * ((len + 127) / 128);\n        struct mxq_cols_ctx",
        "nb = 2 * ((len + 63) / 64);\n        struct mxq_cols_ctx"),
}


def _build(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    p = tmp_path / f"{name}.c"
    p.write_text(src.replace(old, new))
    so = str(tmp_path / f"lib{name}.so")
    import subprocess
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-D_GNU_SOURCE", "-shared", "-fPIC", "-o", so,
                           str(p), "-lm", "-lpthread"])
    return oracle.load(so)


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def pins_pass(lib) -> bool:
    """A compact run of the pins (golden routing, brute-force routing and ties,
    dense brute force in bf16 and fp64, autograd, MXFP8 goldens and torch's
    fp8 cast). True iff every pin holds."""
    try:
        g = json.load(open(os.path.join(GOLD, "route_tiny.json")))
        logits = np.array([[float(v) for v in row] for row in g["logits"]], np.float32)
        r = oracle.route(logits, g["k"], g["tile_m"], lib=lib)
        for key in ("topk_idx", "token_pos", "sorted_token", "sorted_slot", "tile_offsets"):
            if not np.array_equal(r[key], np.array(g[key])):
                return False
        T, d, E, k, h = 40, 16, 4, 2, 16
        inp = dict(logits=synth.normal((T, E), 5, 0, 1.0), x=synth.normal((T, d), 5, 1, 1.0),
                   w1=synth.normal((E, 2 * h, d), 5, 2, 0.2), w2=synth.normal((E, d, h), 5, 3, 0.2),
                   dout=synth.normal((T, d), 5, 4, 1.0))
        for dt in ("bf16", "f64"):
            f = oracle.layer_forward(inp, k, dt, lib=lib)
            b = brute.dense_forward(inp["logits"], inp["x"], inp["w1"], inp["w2"], k, dt)
            if _rel(f["out"], b["out"]) > (1e-2 if dt == "bf16" else 1e-12):
                return False
            e_of = oracle.expert_of_rows(f["route"]["counts"])
            y_b = b["y_all"][e_of, f["route"]["sorted_token"]]
            if dt == "bf16" and (f["y_perm"] != y_b).mean() > 1e-3:
                return False
        f = oracle.layer_forward(inp, k, "f64", lib=lib)
        bw = oracle.layer_backward(inp, f, k, "f64", lib=lib)
        ref = brute.autograd_layer(inp["logits"], inp["x"], inp["w1"], inp["w2"], inp["dout"], k)
        for key, tol in (("dx", 1e-6), ("dW1", 1e-6), ("dW2", 1e-6), ("dlogits", 1e-6)):
            if _rel(bw[key], ref[key]) > tol:
                return False
        gm = json.load(open(os.path.join(GOLD, "e4m3_codes.json")))
        for v, code, _ in gm["encode"]:
            if lib.oracle_e4m3_encode(float(v)) != int(code, 16):
                return False
        for amax, byte, _ in gm["scale"]:
            if lib.oracle_mx_scale(float(np.float32(amax))) != byte:
                return False
        vals = np.random.default_rng(0).standard_normal(4000) * 30
        ours = np.array([lib.oracle_e4m3_encode(float(v)) for v in vals], np.uint8)
        ref8 = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if not np.array_equal(ours, ref8):
            return False
        return _mx_layouts_pass(lib)
    except (AssertionError, ValueError, IndexError):
        return False


def _mx_layouts_pass(lib) -> bool:
    """MXFP8 quantisation in both layouts against the torch-cast round trip,
    with row groups (one empty, a short last block) for the column layout,
    whose padding past a group's rows must hold zero bytes and zero scales."""
    rng = np.random.default_rng(4)
    # magnitudes drawn per element, and an outlier on the diagonal, so that
    # every position of a row block and of a column block is its maximum in
    # some block
    a = rng.standard_normal((70, 64)) * np.exp(rng.uniform(-6, 6, (70, 64)))
    for i in range(64):
        a[i, i] = 1e4 * (1.0 + rng.uniform())
    a = a.astype(np.float32)
    if not np.array_equal(oracle.mx_rows(a, lib=lib), brute.mx_rows_torch(a)):
        return False
    go = np.array([0, 45, 45, 70], np.int32)
    q, sc = oracle.mxfp8_quantize(a, 0, go, lib=lib)
    vals = oracle.mxfp8_dequantize(q, sc, a.shape[0], a.shape[1], 0, go)
    bb = 0
    for g in range(len(go) - 1):
        r0, r1 = int(go[g]), int(go[g + 1])
        nb = 4 * -(-(r1 - r0) // 128)
        if r1 > r0 and not np.array_equal(vals[r0:r1], brute.mx_cols_torch(a[r0:r1])):
            return False
        qg = q[bb * 32 * a.shape[1]:(bb + nb) * 32 * a.shape[1]].reshape(a.shape[1], nb * 32)
        sg = sc[bb * a.shape[1]:(bb + nb) * a.shape[1]].reshape(a.shape[1], nb)
        if np.any(qg[:, r1 - r0:] != 0) or np.any(sg[:, -(-(r1 - r0) // 32):] != 0):
            return False
        bb += nb
    return q.size == bb * 32 * a.shape[1]


def test_unmutated_oracle_passes_the_compact_pins():
    assert pins_pass(oracle.load())


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    lib = _build(tmp_path, name)
    assert not pins_pass(lib), f"planted mistake '{name}' went unnoticed"
