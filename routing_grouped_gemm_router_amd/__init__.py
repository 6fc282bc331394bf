"""Python binding of libmoe, the MI355X MoE expert layer (argument marshalling only).

Every function here has the name of a C entry point in include/moe.h and does
nothing but check tensor shapes/dtypes on the host, pass `data_ptr()`s, sizes
and the current HIP stream to the library, and raise on a non-OK status. All
arithmetic runs in the library's HIP kernels. The library is loaded from this
package's directory; if it is missing, importing the binding raises (there is
no fallback path).

`MoELayer` strings the calls together in the layer's order (route -> permute
-> grouped GEMM + SwiGLU -> grouped GEMM -> combine; `moe_backward`) and owns
the saved tensors and intermediates as torch allocations.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, \
    MOE_ERR_LAUNCH = range(7)
MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_GG_FWD, MOE_GG_DGRAD, MOE_GG_WGRAD = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU_FWD, MOE_EPI_SWIGLU_BWD = 0, 1, 2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {_lib.moe_status_str(status).decode()} (status {status})")
        self.status = status


class GemmDesc(ctypes.Structure):
    _fields_ = [("mode", _I32), ("dtype", _I32), ("epilogue", _I32), ("n_groups", _I32),
                ("rows", _I64), ("M", _I32), ("N", _I32), ("K", _I32),
                ("offsets", _P), ("A", _P), ("B", _P), ("C", _P), ("a_scale", _P),
                ("b_scale", _P), ("aux", _P), ("aux_out", _P), ("aux_out_scale", _P),
                ("ws", _P), ("ws_bytes", _SZ), ("accumulate", _I32), ("aux_out_cols", _P),
                ("aux_out_cols_scale", _P)]


class BwdDesc(ctypes.Structure):
    _fields_ = [("dtype", _I32), ("d", _I32), ("h", _I32), ("E", _I32), ("k", _I32), ("T", _I64),
                ("x_perm", _P), ("ab", _P), ("hp", _P), ("y_perm", _P), ("topk_gate", _P),
                ("topk_idx", _P), ("token_pos", _P), ("offsets", _P), ("w1", _P), ("w2", _P),
                ("dout", _P), ("dx", _P), ("dlogits", _P), ("dw1", _P), ("dw2", _P),
                ("dgate", _P), ("dy_perm", _P), ("dab", _P), ("dx_perm", _P), ("x", _P),
                ("sorted_token", _P), ("w1t", _P), ("w1t_scale", _P), ("w2t", _P),
                ("w2t_scale", _P), ("ws", _P), ("ws_bytes", _SZ), ("accumulate_dw", _I32),
                ("stage_events", ctypes.POINTER(_P)), ("hp_cols", _P), ("hp_cols_scale", _P)]

class CopyWalk(ctypes.Structure):
    _fields_ = [("extent", _I64 * 4), ("copies", _I64), ("zero_copies", _I64),
                ("lowest", _I64 * 4), ("end", _I64 * 4), ("first_bad", _I32),
                ("bad_offset", _I64), ("bad_bytes", _I64)]


class BwdWsLayout(ctypes.Structure):
    _fields_ = [(n, _SZ) for n in ("row_q", "row_s", "col0_q", "col0_s", "col1_q", "col1_s",
                                   "total")]


MOE_BWD_MAX_STAGES = 10
BWD_STAGES = {
    "bf16": ("combine_bwd", "gemm2_dgrad_swiglu", "gemm2_wgrad", "gemm1_dgrad", "unpermute_bwd",
             "gemm1_wgrad"),
    "mxfp8": ("combine_bwd", "quant_dy_both", "gemm2_dgrad_swiglu", "quant_hp_cols", "gemm2_wgrad",
              "quant_dab_both", "gemm1_dgrad", "unpermute_bwd", "quant_x_cols", "gemm1_wgrad"),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m routing_grouped_gemm_router_amd.build` "
            "(the MoE layer has no non-HIP path)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_status_str.argtypes = [_I32]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_version.restype = _I32
    lib.moe_route_workspace_size.argtypes = [_I64, _I32, _I32]
    lib.moe_route_workspace_size.restype = _SZ
    lib.moe_route.argtypes = [_P, _I64, _I32, _I32, _I32] + [_P] * 9 + [_SZ, _P]
    lib.moe_route.restype = _I32
    lib.moe_route_noalloc.argtypes = [_P, _I64, _I32, _I32, _I32] + [_P] * 9
    lib.moe_route_noalloc.restype = _I32
    lib.moe_permute.argtypes = [_P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _P]
    lib.moe_permute.restype = _I32
    lib.moe_combine.argtypes = [_P, _I32, _P, _P, _I64, _I32, _I32, _P, _P]
    lib.moe_combine.restype = _I32
    lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(GemmDesc), _P]
    lib.moe_grouped_gemm.restype = _I32
    lib.moe_grouped_gemm_workspace_size.argtypes = [ctypes.POINTER(GemmDesc)]
    lib.moe_grouped_gemm_workspace_size.restype = _SZ
    lib.moe_backward.argtypes = [ctypes.POINTER(BwdDesc), _P]
    lib.moe_backward.restype = _I32
    lib.moe_backward_workspace_size.argtypes = [ctypes.POINTER(BwdDesc)]
    lib.moe_backward_workspace_size.restype = _SZ
    lib.moe_backward_workspace_layout.argtypes = [ctypes.POINTER(BwdDesc), ctypes.POINTER(BwdWsLayout)]
    lib.moe_backward_workspace_layout.restype = _I32
    lib.moe_gemm_copy_walk.argtypes = [ctypes.POINTER(GemmDesc), _P, ctypes.POINTER(CopyWalk)]
    lib.moe_gemm_copy_walk.restype = _I32
    lib.moe_gemm_hp_store_walk.argtypes = [ctypes.POINTER(GemmDesc), _P, ctypes.POINTER(CopyWalk)]
    lib.moe_gemm_hp_store_walk.restype = _I32
    lib.mxfp8_quantize.argtypes = [_P, _I32, _I64, _I64, _I32, _P, _I32, _P, _P, _P, _P]
    lib.mxfp8_quantize.restype = _I32
    lib.mxfp8_col_blocks.argtypes = [_I64, _I32]
    lib.mxfp8_col_blocks.restype = _SZ
    lib.mxfp8_quantize_both.argtypes = [_P, _I32, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P]
    lib.mxfp8_quantize_both.restype = _I32
    lib.moe_capacity_pad.argtypes = [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _P]
    lib.moe_capacity_pad.restype = _I32
    lib.moe_capacity_zero_rows.argtypes = [_P, _I32, _P, _I32, _I32, _I32, _P]
    lib.moe_capacity_zero_rows.restype = _I32
    lib.moe_load_balance_workspace_size.argtypes = [_I64, _I32]
    lib.moe_load_balance_workspace_size.restype = _SZ
    lib.moe_load_balance.argtypes = [_P, _P, _I64, _I32, _I32, ctypes.c_float, _P, _P, _P, _SZ, _P]
    lib.moe_load_balance.restype = _I32
    return lib


# torch must be imported first so that libmoe binds to the HIP runtime torch
# already loaded (both carry the soname libamdhip64.so.7)
_lib = _load()


def lib():
    return _lib


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.uint8:
        return MOE_MXFP8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on GPU, got "
                         f"{t.dtype} {tuple(t.shape)} (contiguous={t.is_contiguous()}, "
                         f"device={t.device})")


def _need_bytes(t, nbytes, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.uint8 or not t.is_contiguous() or not t.is_cuda or t.numel() < nbytes:
        raise ValueError(f"{name}: expected a contiguous uint8 GPU buffer of at least {nbytes} "
                         f"bytes, got {t.dtype} {tuple(t.shape)}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)


def moe_route_workspace_size(T: int, E: int, k: int) -> int:
    return int(_lib.moe_route_workspace_size(T, E, k))


def moe_route(logits: torch.Tensor, k: int, tile_m: int = 128, out: dict | None = None,
              ws: torch.Tensor | None = None) -> dict:
    """Top-k routing + metadata (see moe.h). Returns a dict of device tensors."""
    T, E = logits.shape
    dev = logits.device
    R = T * k
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(topk_idx=torch.empty((T, k), **i32),
                   topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                   counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                   token_pos=torch.empty((T, k), **i32), sorted_token=torch.empty(R, **i32),
                   sorted_slot=torch.empty(R, **i32), tile_offsets=torch.empty(E + 1, **i32))
    _need(logits, (T, E), torch.float32, "logits")
    wsb = moe_route_workspace_size(T, E, k)
    if ws is None:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check("moe_route", _lib.moe_route(
        _p(logits), T, E, k, tile_m, _p(out["topk_idx"]), _p(out["topk_gate"]), _p(out["counts"]),
        _p(out["offsets"]), _p(out["token_pos"]), _p(out["sorted_token"]), _p(out["sorted_slot"]),
        _p(out["tile_offsets"]), _p(ws), ws.numel(), _stream()))
    return out


MOE_ROUTE_NOALLOC_SCRATCH_BYTES = 4 << 20


def moe_route_noalloc(logits: torch.Tensor, k: int, tile_m: int = 128,
                      out: dict | None = None) -> dict:
    """moe_route with the library's own per-GPU scratch (see moe.h): the C
    call allocates nothing. Pass `out` (as moe_route returns) to avoid the
    output allocations here as well."""
    T, E = logits.shape
    dev = logits.device
    R = T * k
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(topk_idx=torch.empty((T, k), **i32),
                   topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                   counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                   token_pos=torch.empty((T, k), **i32), sorted_token=torch.empty(R, **i32),
                   sorted_slot=torch.empty(R, **i32), tile_offsets=torch.empty(E + 1, **i32))
    _need(logits, (T, E), torch.float32, "logits")
    _check("moe_route_noalloc", _lib.moe_route_noalloc(
        _p(logits), T, E, k, tile_m, _p(out["topk_idx"]), _p(out["topk_gate"]), _p(out["counts"]),
        _p(out["offsets"]), _p(out["token_pos"]), _p(out["sorted_token"]), _p(out["sorted_slot"]),
        _p(out["tile_offsets"]), _stream()))
    return out


def moe_permute(x: torch.Tensor, token_pos: torch.Tensor, x_perm: torch.Tensor | None = None,
                x_scale: torch.Tensor | None = None, x_perm_scale: torch.Tensor | None = None):
    """x_perm[token_pos[t, j]] = x[t]. For MXFP8 pass uint8 x plus x_scale."""
    T, d = x.shape
    k = token_pos.shape[1]
    if x_perm is None:
        x_perm = torch.empty((T * k, d), dtype=x.dtype, device=x.device)
    dt = _dt(x)
    if dt == MOE_MXFP8 and x_perm_scale is None:
        x_perm_scale = torch.empty((T * k, d // 32), dtype=torch.uint8, device=x.device)
    _check("moe_permute", _lib.moe_permute(_p(x), _p(x_scale), dt, T, d, k, _p(token_pos),
                                           _p(x_perm), _p(x_perm_scale), _stream()))
    return (x_perm, x_perm_scale) if dt == MOE_MXFP8 else x_perm


def moe_combine(y_perm: torch.Tensor, topk_gate: torch.Tensor, token_pos: torch.Tensor,
                out: torch.Tensor | None = None) -> torch.Tensor:
    T, k = token_pos.shape
    d = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device)
    _check("moe_combine", _lib.moe_combine(_p(y_perm), _dt(y_perm), _p(topk_gate), _p(token_pos),
                                           T, d, k, _p(out), _stream()))
    return out


def _need_elems(t, n, dtype, name):
    """t is a contiguous GPU tensor of `dtype` with at least n elements."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected a contiguous {dtype} GPU tensor, got {t.dtype} "
                         f"(contiguous={t.is_contiguous()}, device={t.device})")
    if t.numel() < n:
        raise ValueError(f"{name}: needs at least {n} elements, has {t.numel()}")


_TORCH_DT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_MXFP8: torch.uint8}


def _check_gemm_operands(mode, dt, epilogue, A, B, C, offsets, rows, M, N, K, aux, aux_out,
                         a_scale, b_scale, aux_out_scale=None, aux_out_cols=None,
                         aux_out_cols_scale=None):
    """Host-side sizes of every operand against what the mode reads and
    writes (the C ABI sees only pointers, so an undersized tensor would be
    read or written past its end on the device)."""
    E = offsets.numel() - 1
    _need_elems(offsets, E + 1, torch.int32, "offsets")
    hp_quantised = aux_out_scale is not None
    if hp_quantised and (dt != MOE_MXFP8 or epilogue != MOE_EPI_SWIGLU_FWD):
        raise ValueError("aux_out_scale: only the MXFP8 SwiGLU forward stores H' quantised")
    if offsets.device != A.device:
        raise ValueError("offsets must be on A's device")
    et = _TORCH_DT[dt]
    act = torch.bfloat16 if dt == MOE_MXFP8 else et      # stored activations
    if mode == MOE_GG_WGRAD:
        if dt == MOE_MXFP8:
            nb = mxfp8_col_blocks(rows, E)
            _need_elems(A, nb * 32 * M, et, "A")
            _need_elems(B, nb * 32 * N, et, "B")
            _need_elems(a_scale, nb * M, torch.uint8, "a_scale")
            _need_elems(b_scale, nb * N, torch.uint8, "b_scale")
        else:
            _need_elems(A, rows * M, et, "A")
            _need_elems(B, rows * N, et, "B")
        _need_elems(C, E * M * N, torch.float32, "C")
        return
    _need_elems(A, rows * K, et, "A")
    _need_elems(B, E * N * K, et, "B")
    if dt == MOE_MXFP8:
        _need_elems(a_scale, rows * (K // 32), torch.uint8, "a_scale")
        _need_elems(b_scale, E * N * (K // 32), torch.uint8, "b_scale")
    if epilogue == MOE_EPI_SWIGLU_BWD:
        _need_elems(C, rows * 2 * N, act, "C")
        _need_elems(aux, rows * 2 * N, act, "aux")
    else:
        _need_elems(C, rows * N, act, "C")
    if epilogue == MOE_EPI_SWIGLU_FWD:
        if hp_quantised:
            # H' stored as MXFP8 in both layouts instead of bf16
            h, nb = N // 2, mxfp8_col_blocks(rows, E)
            _need_elems(aux_out, rows * h, torch.uint8, "aux_out")
            _need_elems(aux_out_scale, rows * (h // 32), torch.uint8, "aux_out_scale")
            _need_elems(aux_out_cols, nb * 32 * h, torch.uint8, "aux_out_cols")
            _need_elems(aux_out_cols_scale, nb * h, torch.uint8, "aux_out_cols_scale")
        else:
            _need_elems(aux_out, rows * (N // 2), act, "aux_out")


def moe_grouped_gemm(mode: int, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                     offsets: torch.Tensor, epilogue: int = MOE_EPI_NONE, M: int = 0, N: int = 0,
                     K: int = 0, aux: torch.Tensor | None = None,
                     aux_out: torch.Tensor | None = None, a_scale=None, b_scale=None,
                     aux_out_scale=None, dtype: int | None = None, accumulate: bool = False,
                     rows: int | None = None, aux_out_cols=None, aux_out_cols_scale=None):
    """One grouped GEMM (see moe.h for the modes and epilogues). Every
    operand's dtype and size is checked against the mode before the call.
    rows = total routed rows (offsets[-1]); it defaults to A.shape[0] and must
    be given for MXFP8 WGRAD, whose operands are flat column-block arrays.
    MXFP8 SwiGLU forward with aux_out_scale: H' is stored quantised, along h
    into aux_out (uint8 [rows, h]) and aux_out_scale, and along the rows of
    each group into aux_out_cols / aux_out_cols_scale (the layouts
    mxfp8_quantize_both writes)."""
    dt = _dt(A) if dtype is None else dtype
    if dt not in _TORCH_DT:
        raise ValueError(f"unsupported GEMM dtype {dt}")
    if rows is None:
        if mode == MOE_GG_WGRAD and dt == MOE_MXFP8:
            raise ValueError("MXFP8 WGRAD: pass rows (the column-block operands are flat)")
        rows = A.shape[0]
    _check_gemm_operands(mode, dt, epilogue, A, B, C, offsets, rows, M, N, K, aux, aux_out,
                         a_scale, b_scale, aux_out_scale, aux_out_cols, aux_out_cols_scale)
    desc = GemmDesc()
    desc.accumulate = 1 if accumulate else 0
    desc.mode = mode
    desc.dtype = dt
    desc.epilogue = epilogue
    desc.n_groups = offsets.numel() - 1
    desc.rows = rows
    desc.M, desc.N, desc.K = M, N, K
    desc.offsets = offsets.data_ptr()
    desc.A, desc.B, desc.C = A.data_ptr(), B.data_ptr(), C.data_ptr()
    desc.a_scale = a_scale.data_ptr() if a_scale is not None else None
    desc.b_scale = b_scale.data_ptr() if b_scale is not None else None
    desc.aux = aux.data_ptr() if aux is not None else None
    desc.aux_out = aux_out.data_ptr() if aux_out is not None else None
    desc.aux_out_scale = aux_out_scale.data_ptr() if aux_out_scale is not None else None
    desc.aux_out_cols = aux_out_cols.data_ptr() if aux_out_cols is not None else None
    desc.aux_out_cols_scale = (aux_out_cols_scale.data_ptr() if aux_out_cols_scale is not None
                               else None)
    wsb = int(_lib.moe_grouped_gemm_workspace_size(ctypes.byref(desc)))
    ws = torch.empty(wsb, dtype=torch.uint8, device=A.device) if wsb else None
    desc.ws = ws.data_ptr() if ws is not None else None
    desc.ws_bytes = wsb
    _check("moe_grouped_gemm", _lib.moe_grouped_gemm(ctypes.byref(desc), _stream()))
    return C


def moe_backward(saved: dict, dout: torch.Tensor, E: int, k: int, d: int, h: int,
                 out: dict | None = None, want_dgate: bool = True, mxfp8: bool = False,
                 accumulate_dw: bool = False, stage_events=None) -> dict:
    """Backward of the whole layer. `saved` holds the forward tensors
    (x_perm, ab, hp, y_perm, topk_gate, topk_idx, token_pos, offsets, w1, w2;
    with mxfp8: x, sorted_token, w1t, w1t_scale, w2t, w2t_scale instead of
    x_perm, w1, w2)."""
    T = dout.shape[0]
    R = T * k
    dev, dt = dout.device, dout.dtype
    if out is None:
        out = dict(dx=torch.empty((T, d), dtype=dt, device=dev),
                   dlogits=torch.empty((T, E), dtype=torch.float32, device=dev),
                   dw1=torch.empty((E, 2 * h, d), dtype=torch.float32, device=dev),
                   dw2=torch.empty((E, d, h), dtype=torch.float32, device=dev),
                   dgate=torch.empty((T, k), dtype=torch.float32, device=dev) if want_dgate else None,
                   dy_perm=torch.empty((R, d), dtype=dt, device=dev),
                   dab=torch.empty((R, 2 * h), dtype=dt, device=dev),
                   dx_perm=torch.empty((R, d), dtype=dt, device=dev))
    b = BwdDesc()
    b.accumulate_dw = 1 if accumulate_dw else 0
    b.dtype = MOE_MXFP8 if mxfp8 else _dt(dout)
    b.d, b.h, b.E, b.k, b.T = d, h, E, k, T
    names = ("ab", "hp", "y_perm", "topk_gate", "topk_idx", "token_pos", "offsets")
    names += (("x", "sorted_token", "w1t", "w1t_scale", "w2t", "w2t_scale") if mxfp8
              else ("x_perm", "w1", "w2"))
    for name in names:
        if name == "hp" and saved.get(name) is None and mxfp8:
            continue                               # H' brought in its column layout instead
        setattr(b, name, saved[name].data_ptr())
    if mxfp8 and saved.get("hp_cols") is not None:
        b.hp_cols = saved["hp_cols"].data_ptr()
        b.hp_cols_scale = saved["hp_cols_scale"].data_ptr()
    b.dout = dout.data_ptr()
    for name in ("dx", "dlogits", "dw1", "dw2", "dy_perm", "dab", "dx_perm"):
        setattr(b, name, out[name].data_ptr())
    b.dgate = out["dgate"].data_ptr() if out.get("dgate") is not None else None
    wsb = int(_lib.moe_backward_workspace_size(ctypes.byref(b)))
    ws = out.get("_ws")
    if wsb and (ws is None or ws.numel() < wsb):
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        out["_ws"] = ws
    b.ws = ws.data_ptr() if wsb else None
    b.ws_bytes = wsb
    if stage_events is not None:
        # hipEvent_t handles of recorded torch.cuda.Event objects, one per stage
        arr = (_P * MOE_BWD_MAX_STAGES)(*[ctypes.c_void_p(e.cuda_event) if e is not None else None
                                          for e in list(stage_events) +
                                          [None] * (MOE_BWD_MAX_STAGES - len(stage_events))])
        b.stage_events = ctypes.cast(arr, ctypes.POINTER(_P))
    _check("moe_backward", _lib.moe_backward(ctypes.byref(b), _stream()))
    return out


def moe_gemm_copy_walk(mode: int, dtype: int, epilogue: int, offsets, M: int = 0, N: int = 0,
                       K: int = 0, extents=(0, 0, 0, 0)) -> dict:
    """Host-side walk of every copy moe_grouped_gemm would issue (no GPU).
    offsets: host sequence of n_groups + 1 ints; extents: readable bytes of
    A, B, a_scale, b_scale."""
    off = (ctypes.c_int32 * len(offsets))(*[int(v) for v in offsets])
    g = GemmDesc()
    g.mode, g.dtype, g.epilogue = mode, dtype, epilogue
    g.n_groups = len(offsets) - 1
    g.rows = int(offsets[-1])
    g.M, g.N, g.K = M, N, K
    w = CopyWalk()
    for i, x in enumerate(extents):
        w.extent[i] = int(x)
    _check("moe_gemm_copy_walk", _lib.moe_gemm_copy_walk(ctypes.byref(g), off, ctypes.byref(w)))
    return {"copies": w.copies, "zero_copies": w.zero_copies, "lowest": list(w.lowest),
            "end": list(w.end), "first_bad": w.first_bad, "bad_offset": w.bad_offset,
            "bad_bytes": w.bad_bytes}


def moe_gemm_hp_store_walk(offsets, h: int, K: int, extents=(0, 0, 0, 0)) -> dict:
    """Host-side walk of every store of the MXFP8 SwiGLU forward that writes
    H' quantised (no GPU). offsets: host sequence of n_groups + 1 ints;
    extents: writable bytes of aux_out, aux_out_scale, aux_out_cols,
    aux_out_cols_scale."""
    off = (ctypes.c_int32 * len(offsets))(*[int(v) for v in offsets])
    g = GemmDesc()
    g.mode, g.dtype, g.epilogue = MOE_GG_FWD, MOE_MXFP8, MOE_EPI_SWIGLU_FWD
    g.n_groups = len(offsets) - 1
    g.rows = int(offsets[-1])
    g.N, g.K = 2 * h, K
    w = CopyWalk()
    for i, x in enumerate(extents):
        w.extent[i] = int(x)
    _check("moe_gemm_hp_store_walk", _lib.moe_gemm_hp_store_walk(ctypes.byref(g), off,
                                                                 ctypes.byref(w)))
    return {"stores": w.copies, "lowest": list(w.lowest), "end": list(w.end),
            "first_bad": w.first_bad, "bad_offset": w.bad_offset, "bad_bytes": w.bad_bytes}


def moe_backward_workspace_layout(T: int, E: int, k: int, d: int, h: int) -> dict:
    """Byte offsets of the MXFP8 backward's regions inside its workspace."""
    b = BwdDesc()
    b.dtype, b.T, b.E, b.k, b.d, b.h = MOE_MXFP8, T, E, k, d, h
    L = BwdWsLayout()
    _check("moe_backward_workspace_layout",
           _lib.moe_backward_workspace_layout(ctypes.byref(b), ctypes.byref(L)))
    return {n: getattr(L, n) for n, _ in BwdWsLayout._fields_}


def moe_backward_workspace_size(T: int, E: int, k: int, d: int, h: int, dtype: int) -> int:
    b = BwdDesc()
    b.dtype, b.T, b.E, b.k, b.d, b.h = dtype, T, E, k, d, h
    return _lib.moe_backward_workspace_size(ctypes.byref(b))


def mxfp8_col_blocks(rows: int, n_groups: int) -> int:
    return int(_lib.mxfp8_col_blocks(rows, n_groups))


def mxfp8_quantize(x: torch.Tensor, axis: int = 1, group_offsets: torch.Tensor | None = None,
                   q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                   row_map: torch.Tensor | None = None):
    """OCP MXFP8 quantisation (see moe.h). axis=1 returns q [rows, cols] and
    scale [rows, cols/32]; axis=0 returns the flat column-block layout (groups
    padded to 128 rows) sized for the worst case. With row_map, output row r
    quantises x[row_map[r]] (rows = row_map.numel())."""
    rows = x.shape[0] if row_map is None else row_map.numel()
    cols = x.shape[1]
    dev = x.device
    ng = 0 if group_offsets is None else group_offsets.numel() - 1
    if axis == 1:
        q = q if q is not None else torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        scale = scale if scale is not None else torch.empty((rows, cols // 32), dtype=torch.uint8,
                                                            device=dev)
    else:
        nb = mxfp8_col_blocks(rows, max(ng, 1))
        q = q if q is not None else torch.empty(nb * 32 * cols, dtype=torch.uint8, device=dev)
        scale = scale if scale is not None else torch.empty(nb * cols, dtype=torch.uint8, device=dev)
    _check("mxfp8_quantize", _lib.mxfp8_quantize(_p(x), _dt(x), rows, cols, axis,
                                                 _p(group_offsets), ng, _p(row_map), _p(q),
                                                 _p(scale), _stream()))
    return q, scale


def mxfp8_quantize_both(x: torch.Tensor, group_offsets: torch.Tensor | None = None,
                        out: tuple | None = None):
    """Both orientations from one read (see moe.h): returns (q_rows, s_rows)
    as mxfp8_quantize axis=1 and (q_cols, s_cols) as axis=0 with these groups,
    into `out` = (q_rows, s_rows, q_cols, s_cols) when given."""
    rows, cols = x.shape
    dev = x.device
    ng = 0 if group_offsets is None else group_offsets.numel() - 1
    nb = mxfp8_col_blocks(rows, max(ng, 1))
    if out is not None:
        q1, s1, q0, s0 = out
        _need(q1, (rows, cols), torch.uint8, "q_rows")
        _need(s1, (rows, cols // 32), torch.uint8, "s_rows")
        _need_bytes(q0, nb * 32 * cols, "q_cols")
        _need_bytes(s0, nb * cols, "s_cols")
    else:
        q1 = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s1 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        q0 = torch.empty(nb * 32 * cols, dtype=torch.uint8, device=dev)
        s0 = torch.empty(nb * cols, dtype=torch.uint8, device=dev)
    _check("mxfp8_quantize_both", _lib.mxfp8_quantize_both(
        _p(x), _dt(x), rows, cols, _p(group_offsets), ng, _p(q1), _p(s1), _p(q0), _p(s0),
        _stream()))
    return (q1, s1), (q0, s0)


def moe_capacity_pad(route: dict, capacity: int, out: dict | None = None) -> dict:
    """Padded-capacity layout of moe_route's dropless metadata (see moe.h):
    token_pos [T, k] with dropped slots at -1, offsets [E+1] = e * capacity."""
    T, k = route["topk_idx"].shape
    E = route["offsets"].numel() - 1
    dev = route["offsets"].device
    if out is None:
        out = dict(token_pos=torch.empty((T, k), dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev))
    _check("moe_capacity_pad", _lib.moe_capacity_pad(
        _p(route["topk_idx"]), _p(route["token_pos"]), _p(route["offsets"]), T, E, k, capacity,
        _p(out["token_pos"]), _p(out["offsets"]), _stream()))
    return out


def moe_capacity_zero_rows(buf: torch.Tensor, offsets: torch.Tensor, capacity: int) -> torch.Tensor:
    """Zero the unused capacity rows of a [E*capacity, cols] buffer; offsets
    are the dropless ones (see moe.h)."""
    E = offsets.numel() - 1
    _check("moe_capacity_zero_rows", _lib.moe_capacity_zero_rows(
        _p(buf), _dt(buf), _p(offsets), E, capacity, buf.shape[-1], _stream()))
    return buf


# ---------------------------------------------------------------------------
# the layer


# Scratch tensors shared by every recomputing layer of one shape: what a
# layer rebuilds in its backward lives here instead of being held from its
# forward to its backward.
_SCRATCH: dict = {}


def _scratch(name: str, shape, dtype, device) -> torch.Tensor:
    key = (name, tuple(shape), dtype, str(device))
    t = _SCRATCH.get(key)
    if t is None:
        t = _SCRATCH[key] = torch.empty(shape, dtype=dtype, device=device)
    return t


def _nbytes(ts) -> int:
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


MOE_LB_NSTATS = 8
LB_STAT_NAMES = ("loss", "soft_hard_balance", "hard_balance", "soft_balance", "max_load_over_mean",
                 "min_load_over_mean", "count_cv", "empty_experts")


def moe_load_balance_workspace_size(T: int, E: int) -> int:
    return int(_lib.moe_load_balance_workspace_size(T, E))


def moe_load_balance(logits: torch.Tensor, counts: torch.Tensor, k: int, alpha: float,
                     stats: torch.Tensor | None = None, dlogits: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    """Switch-style balancing loss and load statistics (see moe.h); with
    dlogits, its gradient is added into dlogits. Returns the device stats."""
    T, E = logits.shape
    _need(logits, (T, E), torch.float32, "logits")
    _need(counts, (E,), torch.int32, "counts")
    if stats is None:
        stats = torch.empty(MOE_LB_NSTATS, dtype=torch.float32, device=logits.device)
    if dlogits is not None:
        _need(dlogits, (T, E), torch.float32, "dlogits")
    wsb = moe_load_balance_workspace_size(T, E)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=logits.device)
    _check("moe_load_balance", _lib.moe_load_balance(
        _p(logits), _p(counts), T, E, k, float(alpha), _p(stats), _p(dlogits), _p(ws), ws.numel(),
        _stream()))
    return stats


class _Balance:
    """The optional balancing loss of a layer: statistics after routing in
    the forward, its gradient added into dlogits after the backward."""

    def __init__(self, alpha: float):
        self.alpha = alpha
        self.stats = None
        self.ws = None

    def forward(self, logits, counts, k):
        T, E = logits.shape
        if self.stats is None:
            self.stats = torch.empty(MOE_LB_NSTATS, dtype=torch.float32, device=logits.device)
        wsb = max(moe_load_balance_workspace_size(T, E), 4)
        if self.ws is None or self.ws.numel() < wsb:
            self.ws = torch.empty(wsb, dtype=torch.uint8, device=logits.device)
        self.logits, self.counts, self.k = logits, counts, k
        return moe_load_balance(logits, counts, k, self.alpha, stats=self.stats, ws=self.ws)

    def backward(self, dlogits):
        moe_load_balance(self.logits, self.counts, self.k, self.alpha, stats=self.stats,
                         dlogits=dlogits, ws=self.ws)


class MoELayer:
    """Forward and backward of the MoE expert layer through the C ABI.

    Buffers are allocated once per (T, dtype, device) and reused across calls, so a step
    issues only kernel launches (no allocation, no device->host traffic).

    recompute=True trades compute for activation memory (the trade-off the
    Olmo-core 3 report measures, kongchang.com "where the costs are"): the
    layer keeps only y_perm and the routing metadata from its forward to its
    backward. x_perm, A||B and H' are written to scratch shared by all
    recomputing layers of the shape, and the backward rebuilds them (permute,
    then GEMM1 + SwiGLU) before the layer's backward kernels run. The rebuilt
    tensors are bit-identical to the forward's, so are the gradients.

    aux_alpha adds the balancing loss of moe_load_balance: its statistics
    are in `lb_stats` (device) after forward, and backward adds its
    gradient to dlogits."""

    def __init__(self, w1: torch.Tensor, w2: torch.Tensor, k: int, recompute: bool = False,
                 aux_alpha: float | None = None):
        self.w1, self.w2, self.k = w1, w2, k
        self.E, h2, self.d = w1.shape
        self.h = h2 // 2
        self.recompute = recompute
        self.balance = _Balance(aux_alpha) if aux_alpha is not None else None
        self.lb_stats = None
        self._T = None

    def _check_input(self, x, logits):
        if x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError(f"x: expected [T, {self.d}], got {tuple(x.shape)}")
        if x.dtype != self.w1.dtype or self.w2.dtype != self.w1.dtype:
            raise ValueError(f"x ({x.dtype}) and the weights ({self.w1.dtype}, {self.w2.dtype}) "
                             "must share one dtype")
        if x.device != self.w1.device or x.device != self.w2.device or not x.is_cuda:
            raise ValueError("x and the weights must be on the same GPU")
        _need(x, (x.shape[0], self.d), x.dtype, "x")
        _need(logits, (x.shape[0], self.E), torch.float32, "logits")

    def _alloc(self, T, dev, dt):
        key = (T, dt, str(dev))
        if self._T == key:
            return
        E, k, d, h = self.E, self.k, self.d, self.h
        R = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        self.route = dict(topk_idx=torch.empty((T, k), **i32),
                          topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                          counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                          token_pos=torch.empty((T, k), **i32), sorted_token=torch.empty(R, **i32),
                          sorted_slot=torch.empty(R, **i32), tile_offsets=torch.empty(E + 1, **i32))
        self.route_ws = torch.empty(max(moe_route_workspace_size(T, E, k), 1), dtype=torch.uint8,
                                    device=dev)
        own = (lambda name, shape: torch.empty(shape, dtype=dt, device=dev))
        tmp = (lambda name, shape: _scratch(name, shape, dt, dev)) if self.recompute else own
        self.x_perm = tmp("x_perm", (R, d))
        self.ab = tmp("ab", (R, 2 * h))
        self.hp = tmp("hp", (R, h))
        self.y_perm = own("y_perm", (R, d))
        self.out = torch.empty((T, d), dtype=dt, device=dev)
        self.grads = None
        self._T = key

    def _gemm1(self, offsets):
        moe_grouped_gemm(MOE_GG_FWD, self.x_perm, self.w1, self.ab, offsets,
                         MOE_EPI_SWIGLU_FWD, N=2 * self.h, K=self.d, aux_out=self.hp)

    def forward(self, x: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
        self._check_input(x, logits)
        T, d = x.shape
        self._alloc(T, x.device, x.dtype)
        self.x = x
        r = moe_route(logits, self.k, out=self.route, ws=self.route_ws)
        if self.balance is not None:
            self.lb_stats = self.balance.forward(logits, r["counts"], self.k)
        moe_permute(x, r["token_pos"], self.x_perm)
        self._gemm1(r["offsets"])
        moe_grouped_gemm(MOE_GG_FWD, self.hp, self.w2, self.y_perm, r["offsets"], N=d, K=self.h)
        moe_combine(self.y_perm, r["topk_gate"], r["token_pos"], self.out)
        return self.out

    def saved(self) -> dict:
        r = self.route
        return dict(x_perm=self.x_perm, ab=self.ab, hp=self.hp, y_perm=self.y_perm,
                    topk_gate=r["topk_gate"], topk_idx=r["topk_idx"], token_pos=r["token_pos"],
                    offsets=r["offsets"], w1=self.w1, w2=self.w2)

    def held_bytes(self) -> int:
        """Bytes of activations this layer holds from its forward to its
        backward (the input x and the weights are the caller's)."""
        r = self.route
        meta = _nbytes(r.values())
        if self.recompute:
            return meta + _nbytes([self.y_perm])
        return meta + _nbytes([self.x_perm, self.ab, self.hp, self.y_perm])

    def backward(self, dout: torch.Tensor, accumulate_dw: bool = False,
                 stage_events=None) -> dict:
        """accumulate_dw: add this micro-batch's dW1, dW2 to the ones already
        in self.grads (gradient accumulation between optimizer steps).
        stage_events: optional recorded torch.cuda.Event per backward stage
        (moe_bwd_desc.stage_events)."""
        _need(dout, tuple(self.x.shape), self.x.dtype, "dout")
        if self.recompute:
            moe_permute(self.x, self.route["token_pos"], self.x_perm)
            self._gemm1(self.route["offsets"])
        if accumulate_dw and self.grads is None:
            raise ValueError("accumulate_dw needs the gradients of an earlier backward")
        self.grads = moe_backward(self.saved(), dout, self.E, self.k, self.d, self.h,
                                  out=self.grads, accumulate_dw=accumulate_dw,
                                  stage_events=stage_events)
        if self.balance is not None:
            self.balance.backward(self.grads["dlogits"])
        return self.grads


class MoELayerPadded(MoELayer):
    """The padded-capacity alternative the report compares the dropless layer
    against: every expert owns `capacity` rows of [E*capacity, .] buffers,
    rows past an expert's capacity are dropped (no output, no gradient, gates
    not renormalised) and its unused rows are zero. Routing, dispatch, the
    grouped GEMMs, combine and the backward are the dropless layer's own
    kernels, run on the padded metadata, so only the padding differs."""

    def __init__(self, w1: torch.Tensor, w2: torch.Tensor, k: int, capacity: int):
        super().__init__(w1, w2, k)
        self.capacity = capacity

    def _alloc(self, T, dev, dt):
        if self._T == (T, dt, str(dev)):
            return
        super()._alloc(T, dev, dt)
        E, k, d, h, C = self.E, self.k, self.d, self.h, self.capacity
        P = max(E * C, 1)   # capacity 0 drops everything; keep the buffers non-null
        self.pad = dict(token_pos=torch.empty((T, k), dtype=torch.int32, device=dev),
                        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev))
        self.x_perm = torch.empty((P, d), dtype=dt, device=dev)
        self.ab = torch.empty((P, 2 * h), dtype=dt, device=dev)
        self.hp = torch.empty((P, h), dtype=dt, device=dev)
        self.y_perm = torch.empty((P, d), dtype=dt, device=dev)
        self.grads = dict(dx=torch.empty((T, d), dtype=dt, device=dev),
                          dlogits=torch.empty((T, E), dtype=torch.float32, device=dev),
                          dw1=torch.empty((E, 2 * h, d), dtype=torch.float32, device=dev),
                          dw2=torch.empty((E, d, h), dtype=torch.float32, device=dev),
                          dgate=torch.empty((T, k), dtype=torch.float32, device=dev),
                          dy_perm=torch.empty((P, d), dtype=dt, device=dev),
                          dab=torch.empty((P, 2 * h), dtype=dt, device=dev),
                          dx_perm=torch.empty((P, d), dtype=dt, device=dev))

    def forward(self, x: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
        self._check_input(x, logits)
        T, d = x.shape
        C = self.capacity
        self._alloc(T, x.device, x.dtype)
        self.x = x
        r = moe_route(logits, self.k, out=self.route, ws=self.route_ws)
        p = moe_capacity_pad(r, C, out=self.pad)
        moe_permute(x, p["token_pos"], self.x_perm)
        moe_capacity_zero_rows(self.x_perm, r["offsets"], C)
        moe_grouped_gemm(MOE_GG_FWD, self.x_perm, self.w1, self.ab, p["offsets"],
                         MOE_EPI_SWIGLU_FWD, N=2 * self.h, K=d, aux_out=self.hp)
        moe_grouped_gemm(MOE_GG_FWD, self.hp, self.w2, self.y_perm, p["offsets"], N=d, K=self.h)
        moe_combine(self.y_perm, r["topk_gate"], p["token_pos"], self.out)
        return self.out

    def saved(self) -> dict:
        sv = super().saved()
        sv["token_pos"] = self.pad["token_pos"]
        sv["offsets"] = self.pad["offsets"]
        return sv

    def backward(self, dout: torch.Tensor, accumulate_dw: bool = False,
                 stage_events=None) -> dict:
        moe_capacity_zero_rows(self.grads["dy_perm"], self.route["offsets"], self.capacity)
        return super().backward(dout, accumulate_dw, stage_events)


class MoELayerMX:
    """The layer with MXFP8 GEMMs and an MXFP8 dispatch payload.

    fp32 master weights are quantised once per weight update
    (`prepare_weights`), in both orientations: along d / h for the forward
    GEMMs and, per expert, along 2h / d for the backward dgrads. The forward
    quantises x along d before dispatch, so the row-wise dispatch moves E4M3
    bytes plus their scales; GEMM1 writes AB in bf16 and H' already
    quantised, along h for GEMM2 and along rows per expert for GEMM2's weight
    gradient (fuse_hp; with fuse_hp = False GEMM1 writes bf16 H' and a
    separate pass quantises it: the same bytes); y and out stay
    bf16. The backward (moe_backward with MXFP8) quantises its own GEMM
    operands."""

    def __init__(self, w1_master: torch.Tensor, w2_master: torch.Tensor, k: int,
                 recompute: bool = False, aux_alpha: float | None = None):
        self.E, h2, self.d = w1_master.shape
        self.h = h2 // 2
        self.k = k
        self.recompute = recompute
        self.fuse_hp = True
        self.balance = _Balance(aux_alpha) if aux_alpha is not None else None
        self.lb_stats = None
        self.prepare_weights(w1_master, w2_master)
        self._T = None

    def prepare_weights(self, w1: torch.Tensor, w2: torch.Tensor):
        """Re-quantise the fp32 masters, once per optimizer step: each master
        is read once and written in both orientations (mxfp8_quantize_both)."""
        E, d, h = self.E, self.d, self.h
        dev = w1.device
        g1 = torch.arange(0, E + 1, dtype=torch.int32, device=dev) * (2 * h)
        g2 = torch.arange(0, E + 1, dtype=torch.int32, device=dev) * d
        (self.w1q, self.w1s), (self.w1t, self.w1ts) = mxfp8_quantize_both(
            w1.reshape(E * 2 * h, d), g1)
        (self.w2q, self.w2s), (self.w2t, self.w2ts) = mxfp8_quantize_both(
            w2.reshape(E * d, h), g2)

    def _alloc(self, T, dev):
        key = (T, str(dev))
        if self._T == key:
            return
        E, k, d, h = self.E, self.k, self.d, self.h
        R = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.route = dict(topk_idx=torch.empty((T, k), **i32),
                          topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
                          counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                          token_pos=torch.empty((T, k), **i32), sorted_token=torch.empty(R, **i32),
                          sorted_slot=torch.empty(R, **i32), tile_offsets=torch.empty(E + 1, **i32))
        self.route_ws = torch.empty(max(moe_route_workspace_size(T, E, k), 1), **u8)
        # dispatch payload, A||B, H' and its MXFP8 copy: scratch when recomputing
        tmp = ((lambda name, shape, dt: _scratch("mx_" + name, shape, dt, dev)) if self.recompute
               else (lambda name, shape, dt: torch.empty(shape, dtype=dt, device=dev)))
        self.xq = tmp("xq", (T, d), torch.uint8)
        self.xs = tmp("xs", (T, d // 32), torch.uint8)
        self.xpq = tmp("xpq", (R, d), torch.uint8)
        self.xps = tmp("xps", (R, d // 32), torch.uint8)
        self.ab = tmp("ab", (R, 2 * h), torch.bfloat16)
        # H' and its GEMM2 operand are read in the forward only
        self.hp = _scratch("mx_hp", (R, h), torch.bfloat16, dev)
        self.hpq = _scratch("mx_hpq", (R, h), torch.uint8, dev)
        self.hps = _scratch("mx_hps", (R, h // 32), torch.uint8, dev)
        # H' along rows per expert (GEMM2 wgrad's operand), written by GEMM1
        # with GEMM2's; held instead of bf16 H' (when recomputing, the backward
        # quantises the H' it recomputes and these are scratch)
        nb = mxfp8_col_blocks(R, E)
        if not self.recompute:
            self.hpc = torch.empty(nb * 32 * h, **u8)
            self.hpcs = torch.empty(nb * h, **u8)
        else:
            self.hpc = _scratch("mx_hpc", (nb * 32 * h,), torch.uint8, dev)
            self.hpcs = _scratch("mx_hpcs", (nb * h,), torch.uint8, dev)
        self.y_perm = torch.empty((R, d), **bf)
        self.out = torch.empty((T, d), **bf)
        self.grads = None
        self.bwd_ws = None
        self._T = key

    def hp_quantised_in_gemm1(self) -> bool:
        """The forward's GEMM1 stores H' in both MXFP8 layouts (the backward's
        recomputation of GEMM1 stores bf16 H', which moe_backward quantises)."""
        return self.fuse_hp

    def _gemm1(self, x, offsets, token_pos, quantised_hp: bool = False):
        """Quantised dispatch of x and GEMM1 + SwiGLU (forward, and again in
        the backward when recomputing). quantised_hp: H' goes straight to its
        two MXFP8 layouts instead of bf16."""
        mxfp8_quantize(x, 1, q=self.xq, scale=self.xs)
        moe_permute(self.xq, token_pos, self.xpq, x_scale=self.xs, x_perm_scale=self.xps)
        hp = (dict(aux_out=self.hpq, aux_out_scale=self.hps, aux_out_cols=self.hpc,
                   aux_out_cols_scale=self.hpcs) if quantised_hp else dict(aux_out=self.hp))
        moe_grouped_gemm(MOE_GG_FWD, self.xpq, self.w1q, self.ab, offsets, MOE_EPI_SWIGLU_FWD,
                         N=2 * self.h, K=self.d, a_scale=self.xps, b_scale=self.w1s,
                         dtype=MOE_MXFP8, **hp)

    def forward(self, x: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
        if x.dim() != 2 or x.shape[1] != self.d or x.dtype != torch.bfloat16:
            raise ValueError(f"x: expected bf16 [T, {self.d}], got {x.dtype} {tuple(x.shape)}")
        if x.device != self.w1q.device:
            raise ValueError("x and the weights must be on the same GPU")
        _need(x, tuple(x.shape), torch.bfloat16, "x")
        _need(logits, (x.shape[0], self.E), torch.float32, "logits")
        T, d = x.shape
        h = self.h
        self._alloc(T, x.device)
        self.x = x
        r = moe_route(logits, self.k, out=self.route, ws=self.route_ws)
        if self.balance is not None:
            self.lb_stats = self.balance.forward(logits, r["counts"], self.k)
        fused = self.hp_quantised_in_gemm1()
        self._gemm1(x, r["offsets"], r["token_pos"], quantised_hp=fused)
        if not fused:
            self.quantize_hp(r["offsets"])
        moe_grouped_gemm(MOE_GG_FWD, self.hpq, self.w2q, self.y_perm, r["offsets"], N=d, K=h,
                         a_scale=self.hps, b_scale=self.w2s, dtype=MOE_MXFP8)
        moe_combine(self.y_perm, r["topk_gate"], r["token_pos"], self.out)
        return self.out

    def quantize_hp(self, offsets):
        """H' along h for GEMM2 and, unless recomputing (the backward then
        quantises the H' it recomputes), along rows per expert for GEMM2's
        weight gradient, both from one read."""
        if self.recompute:
            mxfp8_quantize(self.hp, 1, q=self.hpq, scale=self.hps)
        else:
            mxfp8_quantize_both(self.hp, offsets, out=(self.hpq, self.hps, self.hpc, self.hpcs))

    def saved(self) -> dict:
        r = self.route
        sv = dict(x=self.x, sorted_token=r["sorted_token"], ab=self.ab, hp=self.hp,
                  y_perm=self.y_perm, topk_gate=r["topk_gate"], topk_idx=r["topk_idx"],
                  token_pos=r["token_pos"], offsets=r["offsets"], w1t=self.w1t,
                  w1t_scale=self.w1ts, w2t=self.w2t, w2t_scale=self.w2ts)
        if not self.recompute:
            sv.update(hp=None, hp_cols=self.hpc, hp_cols_scale=self.hpcs)
        return sv

    def held_bytes(self) -> int:
        """Bytes of activations held from forward to backward (x and the
        weights are the caller's)."""
        meta = _nbytes(self.route.values())
        if self.recompute:
            return meta + _nbytes([self.y_perm])
        return meta + _nbytes([self.ab, self.hpc, self.hpcs, self.y_perm])

    def backward(self, dout: torch.Tensor, accumulate_dw: bool = False,
                 stage_events=None) -> dict:
        """accumulate_dw: add this micro-batch's dW1, dW2 to the ones already
        in self.grads. stage_events: as MoELayer.backward."""
        _need(dout, tuple(self.x.shape), torch.bfloat16, "dout")
        if self.recompute:
            self._gemm1(self.x, self.route["offsets"], self.route["token_pos"])
        if accumulate_dw and self.grads is None:
            raise ValueError("accumulate_dw needs the gradients of an earlier backward")
        self.grads = moe_backward(self.saved(), dout, self.E, self.k, self.d, self.h,
                                  out=self.grads, mxfp8=True, accumulate_dw=accumulate_dw,
                                  stage_events=stage_events)
        if self.balance is not None:
            self.balance.backward(self.grads["dlogits"])
        return self.grads
