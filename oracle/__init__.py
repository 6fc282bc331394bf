"""CPU oracle for the MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, `__graft_entry__.smoke()` and the bench's CPU-baseline leg
may import this package. The product path (the HIP library and its Python
binding) never does, and shares no code with it.

`moe_oracle.c` holds the arithmetic as plain loops (fp64 sums, ascending
order, rounding only where the layer stores a tensor). This module loads it,
and strings its pieces together in the layer's order:

  route -> permute (row gather) -> expert SwiGLU FFN per row -> combine
  backward: combine-bwd + router-bwd -> FFN backward per row -> weight
  gradients per expert -> unpermute-bwd

following the layer the pages describe: tokens each activate a few experts
(Ai2 Olmo-core 3, kongchang.com, "capacity tax"), the selected rows go into
per-expert buffers (bytechap.com, "How it works"; aizyradar.cn, "What
changed"), the experts run on the uneven groups without padding (kongchang.com,
"routing is a systems problem"), which also names the padded-capacity
alternative reproduced by `capacity=`.

Full-size workloads are checked on samples: `layer_sampled` computes the
outputs of chosen tokens and the weight gradients of chosen experts exactly as
the full layer would (every routed row depends only on its token and expert).
"""
from __future__ import annotations

import ctypes
import time
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "moe_oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")

F32, BF16, F64 = 0, 1, 2
_lib = None


def build(force: bool = False, out: str | None = None, defines=()) -> str:
    """Compile moe_oracle.c with gcc into a shared object (defines are -D flags,
    used by the mutation tests to plant mistakes in a private copy)."""
    out = out or _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-shared", "-fPIC", "-o", out + ".tmp",
               _SRC, "-lm", "-lpthread"] + [f"-D{d}" for d in defines]
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _bind(lib):
    lib.oracle_route.argtypes = [_P, _I64, _I32, _I32, _I32] + [_P] * 8
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_rows_fwd.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_rows_bwd.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_wgrad.argtypes = [_I64, _I32, _I32, _P, _P, _P]
    lib.oracle_combine.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P]
    lib.oracle_combine_bwd.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]
    lib.oracle_router_bwd.argtypes = [_I64, _I32, _I32, _P, _P, _P, _P]
    lib.oracle_unpermute_bwd.argtypes = [_I64, _I32, _I32, _I32, _P, _P, _P]
    lib.oracle_mxfp8_quantize.argtypes = [_P, _I64, _I64, _I32, _P, _I32, _P, _P]
    lib.oracle_mxfp8_quantize.restype = ctypes.c_int
    lib.oracle_mxfp8_dequantize.argtypes = [_P, _P, _I64, _I64, _I32, _P, _I32, _P]
    lib.oracle_mxfp8_dequantize.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_mx_scale.argtypes = [ctypes.c_double]
    lib.oracle_mx_scale.restype = ctypes.c_uint8
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """The oracle library (built on first use). `path` loads another build,
    e.g. a deliberately mutated one."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
        _lib.oracle_set_threads(len(os.sched_getaffinity(0)))
    return _lib


def set_threads(n: int):
    load().oracle_set_threads(int(n))


def threads() -> int:
    return load().oracle_get_threads()


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _ptrs(mats):
    """Array of per-expert double* (None for experts not needed)."""
    arr = (ctypes.c_void_p * len(mats))()
    for i, m in enumerate(mats):
        arr[i] = m.ctypes.data if m is not None else None
    return arr


def _dt(dtype: str) -> int:
    return {"f32": F32, "bf16": BF16, "f64": F64}[dtype]


# ---------------------------------------------------------------------------
# pieces


def route(logits, k: int, tile_m: int = 128, lib=None):
    """Top-k routing and the device metadata the layer keeps on the GPU
    (split sizes and per-expert group sizes: kongchang.com, "routing is a
    systems problem")."""
    lib = lib or load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    R = T * k
    o = dict(topk_idx=np.empty((T, k), np.int32), topk_gate=np.empty((T, k), np.float32),
             counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
             token_pos=np.empty((T, k), np.int32), sorted_token=np.empty(R, np.int32),
             sorted_slot=np.empty(R, np.int32), tile_offsets=np.empty(E + 1, np.int32))
    rc = lib.oracle_route(_ptr(logits), T, E, k, tile_m, _ptr(o["topk_idx"]), _ptr(o["topk_gate"]),
                          _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["token_pos"]),
                          _ptr(o["sorted_token"]), _ptr(o["sorted_slot"]), _ptr(o["tile_offsets"]))
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    return o


def expert_of_rows(counts) -> np.ndarray:
    return np.repeat(np.arange(len(counts), dtype=np.int32), np.asarray(counts))


def rows_fwd(x_rows, expert, W1s, W2s, h: int, dtype: str, hp_in=None, lib=None):
    """Expert SwiGLU FFN forward for each routed row: (AB, H', y), all rounded
    to the storage dtype. W1s/W2s are per-expert fp64 matrices (None where no
    row needs that expert)."""
    lib = lib or load()
    x_rows = _c(x_rows, np.float64)
    n, d = x_rows.shape
    ab = np.empty((n, 2 * h)); hp = np.empty((n, h)); y = np.empty((n, d))
    hp_in = None if hp_in is None else _c(hp_in, np.float64)
    lib.oracle_rows_fwd(n, d, h, _dt(dtype), _ptr(x_rows), _ptr(_c(expert, np.int32)),
                        _ptrs(W1s), _ptrs(W2s), _ptr(hp_in), _ptr(ab), _ptr(hp), _ptr(y))
    return ab, hp, y


def rows_bwd(dy_rows, ab_rows, expert, W1s, W2s, h: int, dtype: str, dab_in=None, lib=None):
    """Expert FFN backward per routed row: (dAB, dx_perm), rounded."""
    lib = lib or load()
    dy_rows = _c(dy_rows, np.float64)
    n, d = dy_rows.shape
    dab = np.empty((n, 2 * h)); dx = np.empty((n, d))
    dab_in = None if dab_in is None else _c(dab_in, np.float64)
    lib.oracle_rows_bwd(n, d, h, _dt(dtype), _ptr(_c(expert, np.int32)), _ptrs(W1s), _ptrs(W2s),
                        _ptr(dy_rows), _ptr(_c(ab_rows, np.float64)), _ptr(dab_in), _ptr(dab),
                        _ptr(dx))
    return dab, dx


def wgrad(a_rows, b_rows, lib=None):
    """C = A^T B summed over rows (fp64, ascending), rounded to fp32."""
    lib = lib or load()
    a_rows = _c(a_rows, np.float64); b_rows = _c(b_rows, np.float64)
    n, m = a_rows.shape
    nn = b_rows.shape[1]
    c = np.empty((m, nn))
    lib.oracle_wgrad(n, m, nn, _ptr(a_rows), _ptr(b_rows), _ptr(c))
    return c


def combine(gate, token_pos, y_perm, dtype: str, lib=None):
    lib = lib or load()
    gate = _c(gate, np.float32); token_pos = _c(token_pos, np.int32)
    T, k = gate.shape
    d = y_perm.shape[1]
    out = np.empty((T, d))
    lib.oracle_combine(T, d, k, _dt(dtype), _ptr(gate), _ptr(token_pos),
                       _ptr(_c(y_perm, np.float64)), _ptr(out))
    return out


def combine_bwd(gate, token_pos, dout, y_perm, dtype: str, lib=None):
    lib = lib or load()
    gate = _c(gate, np.float32); token_pos = _c(token_pos, np.int32)
    T, k = gate.shape
    d = dout.shape[1]
    R = y_perm.shape[0]
    dy = np.zeros((R, d)); dg = np.empty((T, k))
    lib.oracle_combine_bwd(T, d, k, _dt(dtype), _ptr(gate), _ptr(token_pos),
                           _ptr(_c(dout, np.float64)), _ptr(_c(y_perm, np.float64)),
                           _ptr(dy), _ptr(dg))
    return dy, dg


def router_bwd(topk_idx, gate, dgate, E: int, lib=None):
    lib = lib or load()
    topk_idx = _c(topk_idx, np.int32); gate = _c(gate, np.float32)
    T, k = gate.shape
    dl = np.empty((T, E))
    lib.oracle_router_bwd(T, E, k, _ptr(topk_idx), _ptr(gate), _ptr(_c(dgate, np.float64)),
                          _ptr(dl))
    return dl


def unpermute_bwd(token_pos, dx_perm, dtype: str, lib=None):
    lib = lib or load()
    token_pos = _c(token_pos, np.int32)
    T, k = token_pos.shape
    d = dx_perm.shape[1]
    dx = np.empty((T, d))
    lib.oracle_unpermute_bwd(T, d, k, _dt(dtype), _ptr(token_pos), _ptr(_c(dx_perm, np.float64)),
                             _ptr(dx))
    return dx


def mxfp8_quantize(a, axis: int, group_offsets=None, lib=None):
    """OCP MXFP8 quantisation (E4M3 elements, one E8M0 scale per 32 along
    `axis`). axis=1 keeps the layout; axis=0 returns the per-group transposed
    layout, each group padded to 128 rows, described in moe_oracle.c. Returns
    (q, scale) as flat uint8 arrays for axis=0 and shaped arrays for axis=1."""
    lib = lib or load()
    a = _c(a, np.float32)
    rows, cols = a.shape
    if axis == 1:
        q = np.empty((rows, cols), np.uint8); s = np.empty((rows, cols // 32), np.uint8)
        go, ng = None, 0
    else:
        go = np.array([0, rows], np.int32) if group_offsets is None else _c(group_offsets, np.int32)
        ng = len(go) - 1
        nb = int(sum(4 * ((go[g + 1] - go[g] + 127) // 128) for g in range(ng)))
        q = np.empty(nb * 32 * cols, np.uint8); s = np.empty(nb * cols, np.uint8)
    rc = lib.oracle_mxfp8_quantize(_ptr(a), rows, cols, axis, _ptr(go), ng, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle_mxfp8_quantize: bad arguments")
    return q, s


def e4m3_decode_table(lib=None) -> np.ndarray:
    lib = lib or load()
    return np.array([lib.oracle_e4m3_decode(i) for i in range(256)], dtype=np.float64)


def mxfp8_dequantize_rowwise(q, scale):
    """Exact values of an axis=1 MXFP8 tensor (fp64)."""
    tab = e4m3_decode_table()
    v = tab[q]
    sc = np.ldexp(1.0, scale.astype(np.int64) - 127)
    return v * np.repeat(sc, 32, axis=1)


# ---------------------------------------------------------------------------
# the layer


def _expert_mats(W, needed):
    return [np.ascontiguousarray(W[e], dtype=np.float64) if e in needed else None
            for e in range(W.shape[0])]


class _Clock:
    """Adds the wall time of each named stage into `timings` (seconds), when
    a dict is given; for reporting where the oracle's time goes."""

    def __init__(self, timings):
        self.t = timings
        self.t0 = time.perf_counter()

    def lap(self, name):
        now = time.perf_counter()
        if self.t is not None:
            self.t[name] = self.t.get(name, 0.0) + now - self.t0
        self.t0 = now


def layer_forward(inp: dict, k: int, dtype: str, tile_m: int = 128, capacity: int | None = None,
                  lib=None, timings: dict | None = None):
    """Full forward of the layer. With `capacity`, each expert keeps only its
    first `capacity` rows in token order and the rest contribute nothing (the
    padded-capacity alternative; gates are not renormalised). `timings`
    (optional dict) receives the wall seconds of each stage."""
    lib = lib or load()
    clk = _Clock(timings)
    logits, x, W1, W2 = inp["logits"], inp["x"], inp["w1"], inp["w2"]
    E = W1.shape[0]
    h = W1.shape[1] // 2
    r = route(logits, k, tile_m, lib)
    clk.lap("route")
    x_perm = np.asarray(x, np.float64)[r["sorted_token"]]
    clk.lap("permute")
    expert = expert_of_rows(r["counts"])
    needed = set(np.unique(expert).tolist())
    W1s, W2s = _expert_mats(W1, needed), _expert_mats(W2, needed)
    ab, hp, y = rows_fwd(x_perm, expert, W1s, W2s, h, dtype, lib=lib)
    clk.lap("expert_ffn_fwd")
    gate = r["topk_gate"]
    keep = None
    if capacity is not None:
        rank = r["token_pos"] - r["offsets"][r["topk_idx"]]
        keep = rank < capacity
        gate = np.where(keep, gate, np.float32(0)).astype(np.float32)
    out = combine(gate, r["token_pos"], y, dtype, lib)
    clk.lap("combine")
    return dict(route=r, x_perm=x_perm, expert=expert, ab=ab, hp=hp, y_perm=y, out=out,
                keep=keep, W1s=W1s, W2s=W2s)


def layer_backward(inp: dict, fwd: dict, k: int, dtype: str, lib=None,
                   timings: dict | None = None):
    """Full backward: dy_perm, dgate, dlogits, dAB, dx_perm, dX, dW1, dW2.
    `timings` (optional dict) receives the wall seconds of each stage."""
    lib = lib or load()
    clk = _Clock(timings)
    r = fwd["route"]
    E = inp["w1"].shape[0]
    h = inp["w1"].shape[1] // 2
    keep = fwd["keep"]
    gate = r["topk_gate"]
    g_eff = gate if keep is None else np.where(keep, gate, np.float32(0)).astype(np.float32)
    dy, dg = combine_bwd(g_eff, r["token_pos"], inp["dout"], fwd["y_perm"], dtype, lib)
    if keep is not None:
        dg = np.where(keep, dg, 0.0)
    dlogits = router_bwd(r["topk_idx"], gate, dg, E, lib)
    clk.lap("combine_bwd_router_bwd")
    dab, dxp = rows_bwd(dy, fwd["ab"], fwd["expert"], fwd["W1s"], fwd["W2s"], h, dtype, lib=lib)
    if keep is not None:
        kept_row = np.zeros(len(dy), bool)
        kept_row[r["token_pos"][keep]] = True
        dab[~kept_row] = 0.0
        dxp[~kept_row] = 0.0
    clk.lap("expert_ffn_dgrad")
    dx = unpermute_bwd(r["token_pos"], dxp, dtype, lib)
    clk.lap("unpermute_bwd")
    off = r["offsets"]
    d = inp["x"].shape[1]
    dW1 = np.zeros((E, 2 * h, d)); dW2 = np.zeros((E, d, h))
    for e in range(E):
        a, b = off[e], off[e + 1]
        dW2[e] = wgrad(dy[a:b], fwd["hp"][a:b], lib)
        dW1[e] = wgrad(dab[a:b], fwd["x_perm"][a:b], lib)
    clk.lap("wgrad")
    return dict(dy_perm=dy, dgate=dg, dlogits=dlogits, dab=dab, dx_perm=dxp, dx=dx,
                dW1=dW1, dW2=dW2)


def layer_sampled(inp: dict, k: int, dtype: str, tokens, experts, tile_m: int = 128,
                  backward: bool = True, lib=None):
    """Outputs of the layer restricted to `tokens` (out, dX, dlogits, dgate)
    and `experts` (dW1, dW2), computed row by row exactly as the full layer
    computes them. Routing is computed in full."""
    lib = lib or load()
    logits, x, W1, W2 = inp["logits"], inp["x"], inp["w1"], inp["w2"]
    E = W1.shape[0]
    h = W1.shape[1] // 2
    d = x.shape[1]
    r = route(logits, k, tile_m, lib)
    tokens = np.asarray(tokens, np.int64)
    experts = np.asarray(experts, np.int64)
    # rows needed: every slot of every sampled token, every row of every sampled expert
    tok_rows = r["token_pos"][tokens].reshape(-1)
    exp_rows = np.concatenate([np.arange(r["offsets"][e], r["offsets"][e + 1]) for e in experts]) \
        if len(experts) else np.zeros(0, np.int64)
    rows = np.unique(np.concatenate([tok_rows, exp_rows]).astype(np.int64))
    expert_all = expert_of_rows(r["counts"])
    expert = expert_all[rows]
    needed = set(np.unique(expert).tolist())
    W1s, W2s = _expert_mats(W1, needed), _expert_mats(W2, needed)
    src = r["sorted_token"][rows]
    slot = r["sorted_slot"][rows]
    x_rows = np.asarray(x, np.float64)[src]
    ab, hp, y = rows_fwd(x_rows, expert, W1s, W2s, h, dtype, lib=lib)
    row_index = {int(p): i for i, p in enumerate(rows)}
    # combine for sampled tokens: y rows are addressed through a compact table
    pos_c = np.array([[row_index[int(p)] for p in r["token_pos"][t]] for t in tokens], np.int32)
    gate_s = r["topk_gate"][tokens]
    out = combine(gate_s, pos_c, y, dtype, lib)
    res = dict(route=r, rows=rows, out=out, ab=ab, hp=hp, y=y)
    if not backward:
        return res
    dout = np.asarray(inp["dout"], np.float64)
    g_row = r["topk_gate"][src, slot].astype(np.float64)
    # dy rows: round(g * dOut[t]) via the combine-bwd routine on a one-slot view
    dy, _ = combine_bwd(g_row.astype(np.float32)[:, None], np.arange(len(rows), dtype=np.int32)[:, None],
                        dout[src], y, dtype, lib)
    _, dg = combine_bwd(gate_s, pos_c, dout[tokens], y, dtype, lib)
    dlogits = router_bwd(r["topk_idx"][tokens], gate_s, dg, E, lib)
    dab, dxp = rows_bwd(dy, ab, expert, W1s, W2s, h, dtype, lib=lib)
    dx = unpermute_bwd(pos_c, dxp, dtype, lib)
    dW1, dW2 = {}, {}
    for e in experts:
        e = int(e)
        sel = np.array([row_index[int(p)] for p in range(r["offsets"][e], r["offsets"][e + 1])],
                       np.int64)
        dW2[e] = wgrad(dy[sel], hp[sel], lib) if len(sel) else np.zeros((d, h))
        dW1[e] = wgrad(dab[sel], x_rows[sel], lib) if len(sel) else np.zeros((2 * h, d))
    res.update(dgate=dg, dlogits=dlogits, dx=dx, dW1=dW1, dW2=dW2, dy=dy, dab=dab, dx_perm=dxp)
    return res


# ---------------------------------------------------------------------------
# MXFP8 layer: every GEMM input is quantised to MXFP8 along that GEMM's
# reduction axis (OCP MX: one E8M0 scale per 32 elements) and used at its
# exact dequantised value; accumulation is fp64; stored tensors are bf16.
# MXFP8 is named for the GEMMs, saved activations and dispatch payload
# (kongchang.com, "caveats behind the numbers").


def mxfp8_dequantize(q, s, rows: int, cols: int, axis: int, group_offsets=None, lib=None):
    """Exact fp64 values, in [rows, cols] order, of mxfp8_quantize's output."""
    lib = lib or load()
    go = None if group_offsets is None else _c(group_offsets, np.int32)
    ng = 0 if go is None else len(go) - 1
    out = np.empty((rows, cols))
    rc = lib.oracle_mxfp8_dequantize(_ptr(_c(q, np.uint8)), _ptr(_c(s, np.uint8)), rows, cols, axis,
                                     _ptr(go), ng, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_mxfp8_dequantize: bad arguments")
    return out


def mx_rows(a, lib=None):
    """Dequantised values of `a` quantised along rows (blocks of 32 columns)."""
    a = np.asarray(a, np.float32)
    q, s = mxfp8_quantize(a, 1, lib=lib)
    return mxfp8_dequantize(q, s, a.shape[0], a.shape[1], 1, lib=lib)


def mx_cols(a, lib=None):
    """Dequantised values of `a` quantised along columns (blocks of 32 rows,
    one group), returned in a's own [rows, cols] layout."""
    a = np.asarray(a, np.float32)
    rows, cols = a.shape
    go = np.array([0, rows], np.int32)
    q, s = mxfp8_quantize(a, 0, go, lib=lib)
    return mxfp8_dequantize(q, s, rows, cols, 0, go, lib=lib)


def mx_cols_dequantize(q, s, group_offsets, cols):
    """Exact values of the column-block layout, back in [rows, cols] order."""
    tab = e4m3_decode_table()
    go = np.asarray(group_offsets, np.int64)
    out = np.zeros((go[-1], cols))
    bb = 0
    for g in range(len(go) - 1):
        n = go[g + 1] - go[g]
        nb = 4 * (-(-n // 128))
        if nb:
            qg = q[bb * 32 * cols:(bb + nb) * 32 * cols].reshape(cols, nb, 32)
            sg = s[bb * cols:(bb + nb) * cols].reshape(cols, nb).astype(np.int64)
            v = tab[qg] * np.ldexp(1.0, sg - 127)[:, :, None]      # [cols, nb, 32]
            out[go[g]:go[g + 1]] = v.reshape(cols, nb * 32)[:, :n].T
        bb += nb
    return out


def _mx_weights_fwd(W1, W2, experts, lib=None):
    """Per expert in `experts`: W1 along d and W2 along h (the forward GEMMs'
    operands), dequantised from the fp32 masters; None for other experts."""
    E = W1.shape[0]
    w1f = [mx_rows(W1[e], lib) if e in experts else None for e in range(E)]
    w2f = [mx_rows(W2[e], lib) if e in experts else None for e in range(E)]
    return w1f, w2f


def _mx_weights_bwd(W1, W2, experts, lib=None):
    """Per expert in `experts`: W1 along 2h and W2 along d (the dgrads'
    operands), dequantised from the fp32 masters; None for other experts."""
    E = W1.shape[0]
    w1b = [mx_cols(W1[e], lib) if e in experts else None for e in range(E)]
    w2b = [mx_cols(W2[e], lib) if e in experts else None for e in range(E)]
    return w1b, w2b


def _gemm2_operand(hp, lib=None):
    """H' quantised along h: what GEMM2 consumes."""
    return mx_rows(hp, lib)


def _expert_chunks(expert, size):
    """(experts, row indices) for blocks of up to `size` distinct experts.
    Each routed row depends only on its token and its expert, so the rows can
    be taken a block at a time with only that block's weights dequantised."""
    uniq = np.unique(expert)
    for i in range(0, len(uniq), size):
        es = uniq[i:i + size]
        yield set(int(e) for e in es), np.flatnonzero(np.isin(expert, es))


def _mx_layer_rows(inp, k, rows, r, lib, backward, chunk=8, progress=None):
    """MXFP8 layer values for the routed rows `rows` (sorted positions): the
    forward (AB, H', y) and, with backward, dy, dAB and dx_perm. `progress`
    (optional callable) gets a line after each block of experts."""
    note = progress or (lambda msg: None)
    W1, W2 = inp["w1"], inp["w2"]
    h = W1.shape[1] // 2
    d = W2.shape[1]
    expert = expert_of_rows(r["counts"])[rows]
    src = r["sorted_token"][rows]
    x = np.asarray(inp["x"], np.float32)
    toks = np.unique(src)
    xq = mx_rows(x[toks], lib)                               # x quantised along d before dispatch
    x_rows = xq[np.searchsorted(toks, src)]
    n = len(rows)
    ab, hp, y = np.empty((n, 2 * h)), np.empty((n, h)), np.empty((n, d))
    for needed, sel in _expert_chunks(expert, chunk):
        w1f, w2f = _mx_weights_fwd(W1, W2, needed, lib)
        ab[sel], hp[sel], _ = rows_fwd(x_rows[sel], expert[sel], w1f, w2f, h, "bf16", lib=lib)
        hq = _gemm2_operand(hp[sel], lib)                    # H' along h for GEMM2
        y[sel] = rows_fwd(x_rows[sel], expert[sel], w1f, w2f, h, "bf16", hp_in=hq, lib=lib)[2]
        note(f"oracle mxfp8 forward: experts {min(needed)}..{max(needed)} done")
    res = dict(rows=rows, expert=expert, src=src, ab=ab, hp=hp, y=y)
    if not backward:
        return res
    dout = np.asarray(inp["dout"], np.float64)
    g_row = r["topk_gate"][src, r["sorted_slot"][rows]]
    # dy rows: round(g * dOut[t]) via the combine-bwd routine on a one-slot view
    dy, _ = combine_bwd(g_row.astype(np.float32)[:, None], np.arange(n, dtype=np.int32)[:, None],
                        dout[src], y, "bf16", lib)
    dyq = mx_rows(dy, lib)                                   # dy along d for GEMM2 dgrad
    dab, dxp = np.empty((n, 2 * h)), np.empty((n, d))
    for needed, sel in _expert_chunks(expert, chunk):
        w1b, w2b = _mx_weights_bwd(W1, W2, needed, lib)
        dab[sel] = rows_bwd(dyq[sel], ab[sel], expert[sel], w1b, w2b, h, "bf16", lib=lib)[0]
        dabq = mx_rows(dab[sel], lib)                        # dAB along 2h for GEMM1 dgrad
        dxp[sel] = rows_bwd(dyq[sel], ab[sel], expert[sel], w1b, w2b, h, "bf16", dab_in=dabq,
                            lib=lib)[1]
        note(f"oracle mxfp8 backward: experts {min(needed)}..{max(needed)} done")
    res.update(dy=dy, dab=dab, dx_perm=dxp)
    return res


def layer_mx(inp: dict, k: int, tokens=None, experts=None, backward: bool = True, lib=None,
             progress=None):
    """The MXFP8 layer, forward (+ backward) for the rows of `tokens` (all if
    None) and the weight gradients of `experts` (all if None). `progress`
    (optional callable) gets a line as each block of experts is done."""
    lib = lib or load()
    logits, x, W1, W2 = inp["logits"], inp["x"], inp["w1"], inp["w2"]
    E = W1.shape[0]
    h = W1.shape[1] // 2
    d = x.shape[1]
    T = logits.shape[0]
    r = route(logits, k, 128, lib)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    experts = np.arange(E) if experts is None else np.asarray(experts, np.int64)
    tok_rows = r["token_pos"][tokens].reshape(-1)
    exp_rows = np.concatenate([np.arange(r["offsets"][e], r["offsets"][e + 1]) for e in experts]) \
        if len(experts) else np.zeros(0, np.int64)
    rows = np.unique(np.concatenate([tok_rows, exp_rows]).astype(np.int64))
    f = _mx_layer_rows(inp, k, rows, r, lib, backward, progress=progress)
    row_index = {int(p): i for i, p in enumerate(rows)}
    pos_c = np.array([[row_index[int(p)] for p in r["token_pos"][t]] for t in tokens], np.int32)
    gate_s = r["topk_gate"][tokens]
    out = combine(gate_s, pos_c, f["y"], "bf16", lib)
    res = dict(route=r, rows=rows, out=out, ab=f["ab"], hp=f["hp"], y=f["y"])
    if not backward:
        return res
    dout = np.asarray(inp["dout"], np.float64)
    src = f["src"]
    dy, dab, dxp = f["dy"], f["dab"], f["dx_perm"]
    _, dg = combine_bwd(gate_s, pos_c, dout[tokens], f["y"], "bf16", lib)
    dlogits = router_bwd(r["topk_idx"][tokens], gate_s, dg, E, lib)
    dx = unpermute_bwd(pos_c, dxp, "bf16", lib)
    xb = np.asarray(x, np.float32)                           # bf16 values of the layer input
    dW1, dW2 = {}, {}
    for e in experts:
        e = int(e)
        sel = np.array([row_index[int(p)] for p in range(r["offsets"][e], r["offsets"][e + 1])],
                       np.int64)
        if len(sel) == 0:
            dW2[e] = np.zeros((d, h)); dW1[e] = np.zeros((2 * h, d))
            continue
        # wgrad operands along rows, blocks restarting at the expert's first row
        dW2[e] = wgrad(mx_cols(dy[sel], lib), mx_cols(f["hp"][sel], lib), lib)
        dW1[e] = wgrad(mx_cols(dab[sel], lib), mx_cols(xb[src[sel]], lib), lib)
        if progress:
            progress(f"oracle mxfp8 weight gradients of expert {e} done")
    res.update(dy=dy, dgate=dg, dlogits=dlogits, dab=dab, dx_perm=dxp, dx=dx, dW1=dW1, dW2=dW2)
    return res


# ---------------------------------------------------------------------------
# load balance (the report's routing section names "token gerrymandering",
# a balancing loss that improves while the expert loads grow more uneven:
# kongchang.com, "routing is a systems problem"; bytechap.com, "What you can
# do"; it prints no formula). The loss is the Switch Transformer balancing
# loss (Fedus, Zoph and Shazeer 2021), with the fraction of routed rows f_e
# counting all k selections of a token.

LB_STATS = ("loss", "soft_hard_balance", "hard_balance", "soft_balance", "max_load_over_mean",
            "min_load_over_mean", "count_cv", "empty_experts")


def load_balance(logits, counts, k: int, alpha: float):
    """fp64: the balancing loss, the load statistics (named in LB_STATS) and
    the loss gradient with respect to the logits, the counts held fixed.
    Returns (stats[8], dlogits[T, E])."""
    logits = np.asarray(logits, np.float64)
    counts = np.asarray(counts, np.float64)
    T, E = logits.shape
    if T == 0:
        return np.zeros(8), np.zeros((0, E))
    # router probabilities: softmax over all E experts of each token
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)                       # mean probability per expert
    f = counts / (T * k)                     # fraction of routed rows per expert
    balance = E * np.dot(f, P)
    loss = alpha * balance
    mean = T * k / E
    stats = np.array([loss, balance, E * np.dot(f, f), E * np.dot(P, P), counts.max() / mean,
                      counts.min() / mean, counts.std() / mean, float((counts == 0).sum())])
    # dL/dlogit_{t,e} = (alpha E / T) * sum_j f_j dp_{t,j}/dlogit_{t,e}
    #                = (alpha E / T) * p_{t,e} (f_e - sum_j p_{t,j} f_j)
    grad = (alpha * E / T) * p * (f[None, :] - (p @ f)[:, None])
    return stats, grad
