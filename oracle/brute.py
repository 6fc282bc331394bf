"""Independent brute-force forms of the layer, for pinning the oracle (tiny sizes only).

TEST INFRASTRUCTURE ONLY; shares nothing with moe_oracle.c beyond the
definitions both restate.

* routing by a full stable sort of every token's logits (descending; a stable
  sort keeps equal logits in ascending expert order) and positions by listing,
  per expert, the tokens that chose it;
* the forward as "run every expert on every token, then mask": out[t] =
  sum over all experts e of gate[t,e] * FFN_e(x[t]) with gate = 0 for experts
  the token did not select -- the dense form of a top-k mixture (kongchang.com,
  "capacity tax": each token activates a few experts of the pool);
* gates as the full softmax renormalised over the selected experts;
* the backward by PyTorch autograd (fp64, CPU) on the dense form.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 (ties to even) of float64 values, as float64."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    big = np.abs(r) > np.ldexp(255.0, 120)
    r = np.where(big, np.copysign(np.inf, x), r)
    return np.where((x == 0) | ~np.isfinite(x), x, r)


def round_store(x, dtype: str):
    if dtype == "f64":
        return np.asarray(x, np.float64)
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    return round_bf16(x)


def route(logits: np.ndarray, k: int, tile_m: int = 128):
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    gate = (ps / ps.sum(axis=1, keepdims=True)).astype(np.float32)
    chosen = np.zeros((T, E), bool)
    np.put_along_axis(chosen, idx.astype(np.int64), True, axis=1)
    counts = chosen.sum(axis=0).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tiles = -(-counts // tile_m)
    tile_offsets = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int32)
    token_pos = np.empty((T, k), np.int32)
    for e in range(E):
        toks = np.flatnonzero(chosen[:, e])
        for rank, t in enumerate(toks):
            j = int(np.flatnonzero(idx[t] == e)[0])
            token_pos[t, j] = offsets[e] + rank
    sorted_token = np.empty(T * k, np.int32)
    sorted_slot = np.empty(T * k, np.int32)
    for t in range(T):
        for j in range(k):
            sorted_token[token_pos[t, j]] = t
            sorted_slot[token_pos[t, j]] = j
    return dict(topk_idx=idx, topk_gate=gate, counts=counts, offsets=offsets,
                tile_offsets=tile_offsets, token_pos=token_pos, sorted_token=sorted_token,
                sorted_slot=sorted_slot)


def dense_forward(logits, x, w1, w2, k: int, dtype: str):
    """out = sum_e mask[t,e] * FFN_e(x[t]), with every expert run on every token."""
    r = route(logits, k)
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E, h2, _ = w1.shape
    h = h2 // 2
    mask = np.zeros((T, E))
    np.put_along_axis(mask, r["topk_idx"].astype(np.int64), r["topk_gate"].astype(np.float64), 1)
    acc = np.zeros((T, d))
    ys = np.empty((E, T, d))
    for e in range(E):
        pre = x @ np.asarray(w1[e], np.float64).T
        a, b = pre[:, :h], pre[:, h:]
        hp = round_store(a / (1.0 + np.exp(-a)) * b, dtype)
        y = round_store(hp @ np.asarray(w2[e], np.float64).T, dtype)
        ys[e] = y
        acc += mask[:, e:e + 1] * y
    return dict(route=r, out=round_store(acc, dtype), y_all=ys)


def autograd_layer(logits, x, w1, w2, dout, k: int):
    """fp64 dense forward + backward by torch autograd on the CPU (no storage
    rounding). Returns out, dX, dW1, dW2, dlogits."""
    import torch

    L = torch.tensor(np.asarray(logits, np.float64), requires_grad=True)
    X = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    W1 = torch.tensor(np.asarray(w1, np.float64), requires_grad=True)
    W2 = torch.tensor(np.asarray(w2, np.float64), requires_grad=True)
    E = W1.shape[0]
    h = W1.shape[1] // 2
    idx = torch.from_numpy(route(np.asarray(logits, np.float32), k)["topk_idx"].astype(np.int64))
    sel = torch.gather(L, 1, idx)
    g = torch.softmax(sel, dim=1)
    mask = torch.zeros(L.shape, dtype=torch.float64).scatter(1, idx, g)
    out = torch.zeros(X.shape, dtype=torch.float64)
    for e in range(E):
        pre = X @ W1[e].T
        a, b = pre[:, :h], pre[:, h:]
        y = (torch.nn.functional.silu(a) * b) @ W2[e].T
        out = out + mask[:, e:e + 1] * y
    D = torch.tensor(np.asarray(dout, np.float64))
    (out * D).sum().backward()
    return dict(out=out.detach().numpy(), dx=X.grad.numpy(), dW1=W1.grad.numpy(),
                dW2=W2.grad.numpy(), dlogits=L.grad.numpy())


# ---------------------------------------------------------------------------
# MXFP8 layer, dense per expert, quantising with torch's float8_e4m3fn cast


def mx_rows_torch(a):
    """OCP MXFP8 round trip along rows (blocks of 32 columns): scale exponent
    floor(log2 amax) - 8 via frexp, clamp [-127, 127]; elements cast by torch
    after clipping to +-448 (torch's cast does not saturate)."""
    import torch
    a = np.asarray(a, np.float64)
    n, c = a.shape
    blk = a.reshape(n, c // 32, 32)
    amax = np.abs(blk).max(axis=2, keepdims=True)
    _, e = np.frexp(amax)
    s = np.clip(e - 1 - 8, -127, 127)
    s = np.where(amax > 0, s, -127)
    v = np.clip(blk * np.ldexp(1.0, -s), -448.0, 448.0)
    qv = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    return (qv * np.ldexp(1.0, s)).reshape(n, c)


def mx_cols_torch(a):
    """Round trip along columns (blocks of 32 rows; a short last block)."""
    a = np.asarray(a, np.float64)
    n, c = a.shape
    pad = -n % 32
    t = np.concatenate([a.T, np.zeros((c, pad))], axis=1)
    return mx_rows_torch(t)[:, :n].T


def mx_layer(logits, x, w1, w2, dout, k: int):
    """Forward and backward of the MXFP8 layer, one expert at a time over the
    tokens that chose it (ascending)."""
    r = route(np.asarray(logits, np.float32), k)
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E, h2, _ = w1.shape
    h = h2 // 2
    idx, gate = r["topk_idx"], r["topk_gate"].astype(np.float64)
    xq = mx_rows_torch(x)
    out = np.zeros((T, d)); dx = np.zeros((T, d)); dg = np.zeros((T, k))
    dW1 = np.zeros((E, h2, d)); dW2 = np.zeros((E, d, h))
    ys, dxs = {}, {}
    for e in range(E):
        toks, slots = np.nonzero(idx == e)
        if len(toks) == 0:
            continue
        pre = xq[toks] @ mx_rows_torch(w1[e]).T
        a, b = pre[:, :h], pre[:, h:]
        ab = round_bf16(pre)
        hp = round_bf16(a / (1 + np.exp(-a)) * b)
        y = round_bf16(mx_rows_torch(hp) @ mx_rows_torch(w2[e]).T)
        g = gate[toks, slots][:, None]
        dy = round_bf16(g * dout[toks])
        dg[toks, slots] = (dout[toks] * y).sum(1)
        dh = mx_rows_torch(dy) @ mx_cols_torch(w2[e])
        aa, bb = ab[:, :h], ab[:, h:]
        sg = 1 / (1 + np.exp(-aa))
        dab = round_bf16(np.concatenate([dh * bb * sg * (1 + aa * (1 - sg)), dh * aa * sg], 1))
        dxe = round_bf16(mx_rows_torch(dab) @ mx_cols_torch(w1[e]))
        dW2[e] = (mx_cols_torch(dy).T @ mx_cols_torch(hp)).astype(np.float32)
        dW1[e] = (mx_cols_torch(dab).T @ mx_cols_torch(x[toks])).astype(np.float32)
        for i, (t, j) in enumerate(zip(toks, slots)):
            ys[(t, j)] = y[i]
            dxs[(t, j)] = dxe[i]
    for t in range(T):
        out[t] = round_bf16(sum(gate[t, j] * ys[(t, j)] for j in range(k)))
        dx[t] = round_bf16(sum(dxs[(t, j)] for j in range(k)))
    s = (gate * dg).sum(1, keepdims=True)
    dlogits = np.zeros((T, E))
    np.put_along_axis(dlogits, idx.astype(np.int64), (gate * (dg - s)).astype(np.float32), 1)
    return dict(out=out, dx=dx, dW1=dW1, dW2=dW2, dlogits=dlogits, dgate=dg)
