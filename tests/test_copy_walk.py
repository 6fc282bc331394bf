"""Every global -> LDS copy of the grouped GEMM stays inside its operand (no
GPU needed).

moe_gemm_copy_walk runs, on the host, the address code the kernels run
(copy_plan.h) over every tile, wave, lane, instruction and K step of a
launch, and reports the lowest and highest byte read from each operand. The
cases cover every copy path the library launches: bf16 FWD (plain and
SwiGLU), DGRAD (plain, and the SwiGLU backward on the other kernel), WGRAD,
and MXFP8 FWD / DGRAD / WGRAD with their scale copies; ragged groups (empty,
one row, a row short of or past a tile, a long tail), and reduction widths
with a half last K step (d % 64 == 32). Extents are the sizes the operand
contract of moe.h gives each operand. The MXFP8 backward's workspace regions
are checked against the sizes of what is quantised into them and against the
reads of the backward's four GEMMs. The stores of the MXFP8 SwiGLU forward
that writes H' quantised are walked the same way (moe_gemm_hp_store_walk,
with the epilogue's own offset code) against its four outputs.
"""
import numpy as np
import pytest

import routing_grouped_gemm_router_amd as moe

FWD, DGRAD, WGRAD = moe.MOE_GG_FWD, moe.MOE_GG_DGRAD, moe.MOE_GG_WGRAD
NONE, SWF, SWB = moe.MOE_EPI_NONE, moe.MOE_EPI_SWIGLU_FWD, moe.MOE_EPI_SWIGLU_BWD
BF16, MX = moe.MOE_BF16, moe.MOE_MXFP8


def _offsets(counts):
    return [0] + np.cumsum(counts).tolist()


# group sizes: empty groups (first, inner, last), a single row, one short of
# and one past a 128-row tile, exact tiles, and a long group
COUNTS = {
    "ragged": [0, 1, 127, 129, 0, 256, 300, 5, 0],
    "tail": [513, 0, 0, 64, 1, 250, 2, 77],
    "one": [3],
    "long": [0, 1000, 0, 31],
}


def _col_blocks(rows, E):
    return moe.mxfp8_col_blocks(rows, E)


def _extents(mode, dt, epi, rows, E, M, N, K):
    """Readable bytes of A, B, a_scale, b_scale by the operand contract."""
    if dt == BF16:
        if mode == WGRAD:
            return (rows * M * 2, rows * N * 2, 0, 0)
        return (rows * K * 2, E * N * K * 2, 0, 0)
    if mode == WGRAD:
        nbc = _col_blocks(rows, E)
        return (nbc * 32 * M, nbc * 32 * N, nbc * M, nbc * N)
    return (rows * K, E * N * K, rows * K // 32, E * N * K // 32)


def _walk(mode, dt, epi, counts, M=0, N=0, K=0, extents=None):
    off = _offsets(counts)
    rows, E = off[-1], len(counts)
    ext = extents or _extents(mode, dt, epi, rows, E, M, N, K)
    return moe.moe_gemm_copy_walk(mode, dt, epi, off, M=M, N=N, K=K, extents=ext), ext


def _in_bounds(r, ext, n_ops):
    assert r["first_bad"] == -1, r
    for i in range(n_ops):
        if r["end"][i]:
            assert r["lowest"][i] >= 0 and r["end"][i] <= ext[i], (i, r, ext)


# (mode, epilogue, N, K) for the row GEMMs; d % 64 == 32 gives a half last K step
ROW_CASES = [
    (FWD, NONE, 256, 128), (FWD, NONE, 96, 160), (FWD, SWF, 2 * 96, 224), (FWD, SWF, 512, 256),
    (DGRAD, NONE, 160, 96), (DGRAD, NONE, 256, 512), (DGRAD, SWB, 96, 160), (DGRAD, SWB, 256, 128),
]


@pytest.mark.parametrize("counts", list(COUNTS))
@pytest.mark.parametrize("mode,epi,N,K", ROW_CASES)
def test_bf16_row_gemm_copies_in_bounds(mode, epi, N, K, counts):
    r, ext = _walk(mode, BF16, epi, COUNTS[counts], N=N, K=K)
    _in_bounds(r, ext, 2)
    assert r["copies"] > 0
    # every row of A is read whole (rows past a group's end read its last row)
    assert r["lowest"][0] == 0 and r["end"][0] == ext[0]
    # a K extent that is not a whole number of 64-element steps takes zeros
    assert (r["zero_copies"] > 0) == (K % 64 != 0)


@pytest.mark.parametrize("counts", list(COUNTS))
@pytest.mark.parametrize("M,N", [(256, 128), (96, 160), (512, 1024), (160, 32)])
def test_bf16_wgrad_copies_in_bounds(M, N, counts):
    r, ext = _walk(WGRAD, BF16, NONE, COUNTS[counts], M=M, N=N)
    _in_bounds(r, ext, 2)
    assert r["end"][0] == ext[0] and r["end"][1] == ext[1]


MX_ROW_CASES = [(FWD, NONE, 256, 128), (FWD, SWF, 512, 384), (FWD, NONE, 128, 512),
                (DGRAD, NONE, 384, 256), (DGRAD, SWB, 128, 512), (DGRAD, NONE, 256, 1024)]


@pytest.mark.parametrize("counts", list(COUNTS))
@pytest.mark.parametrize("mode,epi,N,K", MX_ROW_CASES)
def test_mxfp8_row_gemm_copies_in_bounds(mode, epi, N, K, counts):
    r, ext = _walk(mode, MX, epi, COUNTS[counts], N=N, K=K)
    _in_bounds(r, ext, 4)
    assert r["end"][0] == ext[0] and r["end"][2] == ext[2]


@pytest.mark.parametrize("counts", list(COUNTS))
@pytest.mark.parametrize("M,N", [(256, 128), (384, 512), (128, 1024), (1024, 256)])
def test_mxfp8_wgrad_copies_in_bounds(M, N, counts):
    r, ext = _walk(WGRAD, MX, NONE, COUNTS[counts], M=M, N=N)
    _in_bounds(r, ext, 4)


def test_full_size_workloads_in_bounds():
    """The bench's shapes: e128_bf16 (R = 65,536, d = 2048, h = 1024) for all
    six roles and the e128_mxfp8 GEMM1 roles (d = 4096, h = 2048), groups
    of 449..567 rows."""
    rng = np.random.default_rng(0)
    counts = rng.multinomial(65536, [1 / 128] * 128).tolist()
    d, h = 2048, 1024
    for mode, epi, M, N, K in [(FWD, SWF, 0, 2 * h, d), (FWD, NONE, 0, d, h), (DGRAD, SWB, 0, h, d),
                               (WGRAD, NONE, d, h, 0), (DGRAD, NONE, 0, d, 2 * h),
                               (WGRAD, NONE, 2 * h, d, 0)]:
        r, ext = _walk(mode, BF16, epi, counts, M=M, N=N, K=K)
        _in_bounds(r, ext, 2)
    counts = rng.multinomial(131072, [1 / 128] * 128).tolist()
    d, h = 4096, 2048
    for mode, epi, M, N, K in [(FWD, SWF, 0, 2 * h, d), (WGRAD, NONE, 2 * h, d, 0)]:
        r, ext = _walk(mode, MX, epi, counts, M=M, N=N, K=K)
        _in_bounds(r, ext, 4)


@pytest.mark.parametrize("dt,mode,epi,M,N,K", [(BF16, DGRAD, NONE, 0, 160, 96),
                                               (BF16, WGRAD, NONE, 96, 160, 0),
                                               (MX, FWD, SWF, 0, 512, 384),
                                               (MX, WGRAD, NONE, 384, 512, 0)])
def test_walk_flags_a_short_operand(dt, mode, epi, M, N, K):
    """The walk is not vacuous: one byte less of any operand it reads to the
    end is reported as the first out-of-bounds read."""
    counts = COUNTS["ragged"]
    r, ext = _walk(mode, dt, epi, counts, M=M, N=N, K=K)
    _in_bounds(r, ext, 4)
    for op in range(4):
        if r["end"][op] != ext[op] or ext[op] == 0:
            continue
        short = list(ext)
        short[op] -= 1
        r2, _ = _walk(mode, dt, epi, counts, M=M, N=N, K=K, extents=short)
        assert r2["first_bad"] == op, (op, r2)
        assert r2["bad_offset"] + r2["bad_bytes"] > short[op]


def test_walk_rejects_bad_offsets_and_f32():
    with pytest.raises(moe.MoeError) as e:
        moe.moe_gemm_copy_walk(FWD, BF16, NONE, [0, 5, 3], N=128, K=128, extents=(1 << 30,) * 4)
    assert e.value.status == moe.MOE_ERR_SHAPE
    with pytest.raises(moe.MoeError) as e:
        moe.moe_gemm_copy_walk(FWD, moe.MOE_F32, NONE, [0, 5], N=128, K=128, extents=(1 << 30,) * 4)
    assert e.value.status == moe.MOE_ERR_DTYPE


# ---------------------------------------------------------------------------
# the MXFP8 backward's workspace


BWD_SHAPES = [  # T, E, k, d, h
    (512, 8, 2, 256, 128),      # h < d, 2h = d
    (300, 8, 2, 128, 256),      # h > d (the case that once overran)
    (1000, 16, 4, 384, 640),    # 2h > d > h
    (64, 256, 8, 128, 128),     # many empty groups
    (1, 4, 4, 256, 512),
    (32768, 128, 4, 4096, 2048),  # the bench's MXFP8 workload
]


@pytest.mark.parametrize("T,E,k,d,h", BWD_SHAPES)
def test_mxfp8_backward_workspace_regions(T, E, k, d, h):
    L = moe.moe_backward_workspace_layout(T, E, k, d, h)
    assert L["total"] == moe.moe_backward_workspace_size(T, E, k, d, h, MX)
    order = [L[n] for n in ("row_q", "row_s", "col0_q", "col0_s", "col1_q", "col1_s", "total")]
    assert order[0] == 0 and all(a <= b for a, b in zip(order, order[1:]))
    assert all(v % 256 == 0 for v in order)
    R = T * k
    nbc = _col_blocks(R, E)
    size = {n: b - a for n, a, b in zip(("row_q", "row_s", "col0_q", "col0_s", "col1_q", "col1_s"),
                                        order, order[1:])}
    # what the backward quantises into each region (mxfp8_quantize's output sizes)
    for w in (d, 2 * h):                       # dy along d, then dAB along 2h: row blocks
        assert size["row_q"] >= R * w and size["row_s"] >= R * w // 32, w
    for w in (d, 2 * h):                       # dy, then dAB: column blocks per expert
        assert size["col0_q"] >= nbc * 32 * w and size["col0_s"] >= nbc * w, w
    for w in (h, d):                           # H', then the gathered x rows
        assert size["col1_q"] >= nbc * 32 * w and size["col1_s"] >= nbc * w, w


@pytest.mark.parametrize("T,E,k,d,h", BWD_SHAPES[:5])
def test_mxfp8_backward_gemm_reads_stay_in_their_regions(T, E, k, d, h):
    L = moe.moe_backward_workspace_layout(T, E, k, d, h)
    rng = np.random.default_rng(T + E)
    R = T * k
    counts = rng.multinomial(R, [1 / E] * E).tolist()
    off = _offsets(counts)
    rq, rs = L["row_s"] - L["row_q"], L["col0_q"] - L["row_s"]
    c0q, c0s = L["col0_s"] - L["col0_q"], L["col1_q"] - L["col0_s"]
    c1q, c1s = L["col1_s"] - L["col1_q"], L["total"] - L["col1_s"]
    gemms = [  # mode, epi, M, N, K, extents (A, B, a_scale, b_scale)
        (DGRAD, SWB, 0, h, d, (rq, E * h * d, rs, E * h * d // 32)),            # dy . W2t
        (WGRAD, NONE, d, h, 0, (c0q, c1q, c0s, c1s)),                           # dW2 = dy^T H'
        (DGRAD, NONE, 0, d, 2 * h, (rq, E * d * 2 * h, rs, E * d * 2 * h // 32)),  # dAB . W1t
        (WGRAD, NONE, 2 * h, d, 0, (c0q, c1q, c0s, c1s)),                       # dW1 = dAB^T x
    ]
    for mode, epi, M, N, K, ext in gemms:
        r = moe.moe_gemm_copy_walk(mode, MX, epi, off, M=M, N=N, K=K, extents=ext)
        _in_bounds(r, ext, 4)


# The MXFP8 SwiGLU forward that stores H' quantised: every store of its
# epilogue, walked on the host with the offsets the kernel computes
# (moe_gemm_hp_store_walk), lies inside the four outputs at the sizes the
# binding requires, and the stores reach exactly the bytes the layouts hold:
# every row of H' along h, and every 128-row unit of every group (padding
# rows included) of the column-block layout.
@pytest.mark.parametrize("name", sorted(COUNTS))
@pytest.mark.parametrize("h", [128, 160, 2048])
def test_hp_store_walk_in_bounds(name, h):
    counts = COUNTS[name]
    off = _offsets(counts)
    R, E = off[-1], len(counts)
    nb = moe.mxfp8_col_blocks(R, E)
    ext = (R * h, R * (h // 32), nb * 32 * h, nb * h)
    w = moe.moe_gemm_hp_store_walk(off, h, 128, ext)
    assert w["first_bad"] == -1, w
    units = sum(-(-c // 128) for c in counts)
    if R == 0:
        assert w["stores"] == 0
        return
    # rows layout: all R rows x h bytes, scales R x h/32
    assert w["lowest"][0] == 0 and w["end"][0] == R * h
    assert w["lowest"][1] == 0 and w["end"][1] == R * (h // 32)
    # column layout: 4 * units blocks of 32 rows per hidden unit
    assert w["lowest"][2] == 0 and w["end"][2] == 4 * units * 32 * h
    assert w["lowest"][3] == 0 and w["end"][3] == 4 * units * h
    # stores per 32 x 32 block of a 128-row unit: 64 lanes x 1 column piece,
    # 32 column scales; rows: 8 x 4 bytes and one scale per row
    n_tiles_h = h // 32
    col_stores = units * 4 * n_tiles_h * (64 + 32)
    row_stores = R * n_tiles_h * (8 + 1)
    assert w["stores"] == col_stores + row_stores


def test_hp_store_walk_catches_short_outputs():
    """A column layout one byte short (or rows one short) is reported."""
    off = _offsets(COUNTS["ragged"])
    R, E, h = off[-1], len(COUNTS["ragged"]), 128
    units = sum(-(-c // 128) for c in COUNTS["ragged"])
    full = (R * h, R * (h // 32), 4 * units * 32 * h, 4 * units * h)
    for i in range(4):
        ext = list(full)
        ext[i] -= 1
        w = moe.moe_gemm_hp_store_walk(off, h, 128, ext)
        assert w["first_bad"] == i, (i, w)
    bad = list(off)
    bad[2], bad[3] = bad[3], bad[2]                                       # offsets decrease
    with pytest.raises(moe.MoeError):
        moe.moe_gemm_hp_store_walk(bad, h, 128, full)
