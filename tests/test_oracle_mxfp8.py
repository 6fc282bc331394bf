"""Pins for the oracle's MXFP8 quantiser (OCP Microscaling v1.0: E4M3
elements, one E8M0 scale per 32 elements -- the format the pages name:
kongchang.com, "caveats behind the numbers")."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_codes():
    g = json.load(open(os.path.join(GOLD, "e4m3_codes.json")))
    lib = oracle.load()
    for v, code, why in g["encode"]:
        v = float(v)
        assert lib.oracle_e4m3_encode(v) == int(code, 16), (v, why)
    for amax, byte, why in g["scale"]:
        assert lib.oracle_mx_scale(float(np.float32(amax))) == byte, (amax, why)


def test_decode_table_against_torch_fp8():
    """Every E4M3 code decodes to torch.float8_e4m3fn's value (a library routine)."""
    tab = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert np.array_equal(tab[~nan], ref[~nan])


def test_all_bf16_inputs_unit_scale_against_torch():
    """All 2^16 bf16 bit patterns through the element encoder at scale 2^0,
    against torch's float->float8_e4m3fn cast (round to nearest even); torch
    does not saturate, so beyond 448 we check the saturation rule directly."""
    lib = oracle.load()
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    vals = bits.double().numpy()
    ours = np.array([lib.oracle_e4m3_encode(float(v)) for v in vals], np.uint8)
    finite = np.isfinite(vals)
    small = finite & (np.abs(vals) < 448)
    ref = torch.from_numpy(vals[small].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[small], ref)
    big = finite & (np.abs(vals) >= 448)
    assert np.all((ours[big] & 0x7F) == 0x7E)
    assert np.all((ours[big] >> 7) == np.signbit(vals[big]))
    assert np.all((ours[np.isnan(vals)] & 0x7F) == 0x7F)


def _blocks(rng, n):
    return (rng.standard_normal((n, 32)) * np.exp(rng.uniform(-20, 20, (n, 1)))).astype(np.float32)


def test_block_properties():
    """Powers of two round-trip exactly; normal-range elements are within
    2^-4 relative; the block max never exceeds 448 * 2^scale... except by
    saturation, which clips at most 12.5% (values in (448, 512) -> 448)."""
    rng = np.random.default_rng(0)
    a = _blocks(rng, 400)
    q, s = oracle.mxfp8_quantize(a, 1)
    v = oracle.mxfp8_dequantize_rowwise(q, s)
    sc = np.ldexp(1.0, s.astype(np.int64) - 127)[:, :1]
    amax = np.abs(a).max(1, keepdims=True)
    assert np.all(amax / sc < 512)
    assert np.all(amax / sc >= 256)
    normal = np.abs(a) / sc >= 2.0 ** -6
    rel = np.abs(v - a) / np.abs(a)
    assert np.all(rel[normal & (np.abs(a) / sc <= 448)] <= 2.0 ** -4)
    clipped = np.abs(a) / sc > 448
    assert np.all(np.abs(v[clipped]) == 448 * np.broadcast_to(sc, a.shape)[clipped])
    p2 = np.ldexp(1.0, rng.integers(-30, 30, (50, 32))).astype(np.float32)
    q2, s2 = oracle.mxfp8_quantize(p2, 1)
    # powers of two within 2^-9 .. 2^8 of the block scale are exact
    v2 = oracle.mxfp8_dequantize_rowwise(q2, s2)
    sc2 = np.ldexp(1.0, s2.astype(np.int64) - 127)[:, :1]
    ok = p2 / sc2 >= 2.0 ** -9
    assert np.array_equal(v2[ok], p2[ok])


def test_special_blocks():
    zero = np.zeros((1, 32), np.float32)
    q, s = oracle.mxfp8_quantize(zero, 1)
    assert s[0, 0] == 0 and np.all(q == 0)
    b = np.zeros((1, 32), np.float32); b[0, 3] = 500.0; b[0, 4] = -1.0
    q, s = oracle.mxfp8_quantize(b, 1)
    assert s[0, 0] == 127 and q[0, 3] == 0x7E and q[0, 4] == 0xB8
    sub = np.full((1, 32), 1e-40, np.float32)
    q, s = oracle.mxfp8_quantize(sub, 1)
    assert s[0, 0] == 0


@pytest.mark.parametrize("groups", [[0, 64], [0, 40, 40, 77, 141], [0, 1, 33, 33, 100]])
def test_axis0_grouped_layout(groups):
    """Column blocks restart at each group; a group of exactly whole blocks equals
    the row-wise quantisation of its transpose; tails are zero-padded to 128 rows."""
    rng = np.random.default_rng(2)
    rows = groups[-1]
    cols = 64
    a = rng.standard_normal((rows, cols)).astype(np.float32)
    go = np.array(groups, np.int32)
    q, s = oracle.mxfp8_quantize(a, 0, go)
    bb = 0
    for g in range(len(go) - 1):
        lo, hi = go[g], go[g + 1]
        n = hi - lo
        nb = 4 * (-(-n // 128))
        if nb == 0:
            continue
        seg = np.zeros((cols, nb * 32), np.float32)
        seg[:, :n] = a[lo:hi].T
        qr, sr = oracle.mxfp8_quantize(seg, 1)
        qg = q[bb * 32 * cols:(bb + nb) * 32 * cols].reshape(cols, nb * 32)
        sg = s[bb * cols:(bb + nb) * cols].reshape(cols, nb)
        assert np.array_equal(qg, qr) and np.array_equal(sg, sr)
        assert np.all(qg[:, n:] == 0)
        bb += nb
    assert len(s) == bb * cols


def test_quantise_bytes_independent_of_threads():
    """The quantiser splits blocks over threads; each block is written by one
    thread, so the bytes are the same for any thread count."""
    a = (np.random.default_rng(3).standard_normal((300, 160)) *
         np.exp(np.random.default_rng(4).uniform(-6, 6, (300, 1)))).astype(np.float32)
    go = np.array([0, 7, 7, 130, 300], np.int32)
    n0 = oracle.threads()
    try:
        res = []
        for n in (1, 5):
            oracle.set_threads(n)
            res.append((oracle.mxfp8_quantize(a, 1), oracle.mxfp8_quantize(a, 0, go)))
    finally:
        oracle.set_threads(n0)
    for (q1, s1), (q2, s2) in zip(res[0], res[1]):
        assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_dequantize_matches_numpy_forms():
    """The C dequantiser against the numpy decode-table forms of both layouts
    (row blocks; column blocks with groups, a short last block, an empty group)."""
    a = (np.random.default_rng(5).standard_normal((260, 96)) *
         np.exp(np.random.default_rng(6).uniform(-20, 20, (260, 1)))).astype(np.float32)
    q, s = oracle.mxfp8_quantize(a, 1)
    assert np.array_equal(oracle.mxfp8_dequantize(q, s, 260, 96, 1),
                          oracle.mxfp8_dequantize_rowwise(q, s))
    go = np.array([0, 33, 33, 200, 260], np.int32)
    q, s = oracle.mxfp8_quantize(a, 0, go)
    assert np.array_equal(oracle.mxfp8_dequantize(q, s, 260, 96, 0, go),
                          oracle.mx_cols_dequantize(q, s, go, 96))
