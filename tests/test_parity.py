"""GPU parity: libgemmf16 (through its C-ABI) against the CPU oracle on the
same seeded inputs.

Acceptance (from the oracle's contract): bit-exact on integer inputs in
[-4, 4] with K <= 128 (every partial sum is an integer of magnitude <= 2048,
exact in fp32 and fp16); elementwise |C_gpu - C_oracle| <= 1e-2 + 2e-3|C_oracle|
on U(-1, 1) inputs.  Every kernel family is forced on every shape it accepts;
inputs are passed as views into NaN-filled buffers where the layout allows,
so any read outside a view turns an output into NaN; outputs are pre-filled
with NaN and surrounded by canaries, so a missing or stray write is seen.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (CANARY, DEV, NAN16, ORACLE_THREADS, Out, assert_bits_equal, assert_close,
                      band_rows, dev_nan, full_size_check, place, say, to_dev, to_host, val)

pytestmark = pytest.mark.gpu

def run(a, b, out=None, **kw):
    say(f"gemm M={a.shape[0]} N={b.shape[1]} K={a.shape[1]} a.stride={a.stride()} "
        f"b.stride={b.stride()} opts={kw}")
    o = out.view if out is not None else None
    c = g.gemm(a, b, out=o, **kw)
    torch.cuda.synchronize()
    return out.result() if out is not None else to_host(c)


def reference(A, B, rows=None):
    """Oracle on the logical row-major host matrices (all rows or some)."""
    K, N = B.shape
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (N, 1), A.shape[0], N, K, nthreads=ORACLE_THREADS)


def check(gpu, ref, mode, what):
    if mode == "int":
        assert_bits_equal(gpu, ref, what)
    else:
        assert_close(gpu, ref, what)


VARIANTS = [dict(variant="auto"), dict(variant="main"), dict(variant="tile64x32"),
            dict(variant="splitk", split_k=2), dict(variant="splitk", split_k=3),
            dict(variant="splitk", split_k=7), dict(variant="main", panel=-1),
            dict(variant="main", panel=1), dict(variant="main", tile=3),
            dict(variant="main", tile=6), dict(variant="splitk", tile=6, split_k=3),
            dict(variant="main", tile=13), dict(variant="splitk", tile=13, split_k=2),
            dict(variant="main", tile=14), dict(variant="splitk", tile=14, split_k=3),
            dict(variant="main", tile=7), dict(variant="splitk", tile=7, split_k=2),
            dict(variant="main", tile=8), dict(variant="splitk", tile=8, split_k=3)]


# ------------------------------------------------------------------ the edge case

@pytest.mark.parametrize("mode", ["uniform", "int"])
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_edge_130x70x65(mode, b_layout):
    M, N, K = 130, 70, 65
    seed = 1001 if mode == "uniform" else 1002
    A = synth.matrix(M, K, seed, synth.TENSOR_A, mode)
    B = synth.matrix(K, N, seed, synth.TENSOR_B, mode)
    ref = reference(A, B)
    a, b = place(A, "row"), place(B, b_layout)
    for kw in VARIANTS:
        out = Out(M, N, ldc=N + 5)
        check(run(a, b, out, **kw), ref, mode, f"130x70x65 {mode} B={b_layout} {kw}")
    p = g.plan(a, b, variant="tile64x32")
    assert (p["tile_m"], p["tile_n"], p["tile_k"], p["grid"]) == (64, 32, 32, 9)
    with pytest.raises(g.GemmError):
        g.gemm(a, b, variant="skinny")          # skinny is for M <= 64


# ------------------------------------------------------------------ layouts and ragged tails

LAYOUT_SHAPES = [(300, 200, 128), (257, 136, 120), (96, 1000, 64), (1000, 24, 128),
                 (129, 129, 127), (64, 72, 131)]


@pytest.mark.parametrize("shape", LAYOUT_SHAPES)
@pytest.mark.parametrize("a_layout,b_layout", [("row", "row"), ("row", "col"), ("col", "row"),
                                               ("col", "col")])
def test_layouts_integer_exact(shape, a_layout, b_layout):
    M, N, K = shape
    A = synth.matrix(M, K, 7, synth.TENSOR_A, "int")
    B = synth.matrix(K, N, 7, synth.TENSOR_B, "int")
    ref = reference(A, B)
    for pad in [(0, 0), (3, 8)]:
        a, b = place(A, a_layout, pad), place(B, b_layout, pad)
        for kw in VARIANTS:
            check(run(a, b, Out(M, N, ldc=N + 3), **kw), ref, "int",
                  f"{shape} A={a_layout} B={b_layout} pad={pad} {kw}")


def test_layout_paths_are_exercised():
    A = synth.matrix(300, 128, 7, 0, "int")
    B = synth.matrix(128, 200, 7, 1, "int")
    seen = set()
    for al in ("row", "col"):
        for bl in ("row", "col"):
            for pad in [(0, 0), (3, 8), (0, 3)]:
                p = g.plan(place(A, al, pad), place(B, bl, pad))
                seen.add((p["a_path"], p["b_path"]))
    assert {"kvec", "rvec", "gather"} <= {x for pair in seen for x in pair}


@pytest.mark.parametrize("shape", [(300, 200, 1000), (257, 136, 777), (513, 260, 2051)])
@pytest.mark.parametrize("a_layout,b_layout", [("row", "row"), ("row", "col"), ("col", "row")])
def test_layouts_uniform(shape, a_layout, b_layout):
    M, N, K = shape
    A = synth.matrix(M, K, 11, synth.TENSOR_A)
    B = synth.matrix(K, N, 11, synth.TENSOR_B)
    ref = reference(A, B)
    a, b = place(A, a_layout, (2, 8)), place(B, b_layout, (1, 8))
    for kw in VARIANTS:
        check(run(a, b, Out(M, N), **kw), ref, "uniform", f"{shape} {a_layout}/{b_layout} {kw}")


def test_tiny_shapes_brute_force():
    sizes = [1, 2, 3, 5, 8, 13]
    for M in sizes:
        for N in sizes:
            for K in sizes:
                A = synth.matrix(M, K, 100 + M, 0, "int")
                B = synth.matrix(K, N, 200 + N, 1, "int")
                ref = reference(A, B)
                a, b = place(A, "row", (1, 2)), place(B, "col", (1, 2))
                for kw in (dict(variant="auto"), dict(variant="main"),
                           dict(variant="tile64x32"), dict(variant="splitk", split_k=2)):
                    check(run(a, b, Out(M, N), **kw), ref, "int", f"{M}x{N}x{K} {kw}")
                if M <= 64:
                    check(run(a, b, Out(M, N), variant="skinny"), ref, "int", f"{M}x{N}x{K} skinny")


# ------------------------------------------------------------------ square sweep

@pytest.mark.parametrize("n", [256, 1024])
def test_square_full(n):
    A = synth.matrix(n, n, 2000 + n, 0)
    B = synth.matrix(n, n, 2000 + n, 1)
    ref = reference(A, B)
    a, b = to_dev(A), to_dev(B)
    for kw in (dict(variant="auto"), dict(variant="main"), dict(variant="splitk", split_k=4)):
        check(run(a, b, Out(n, n), **kw), ref, "uniform", f"square {n} {kw}")


@pytest.mark.parametrize("n", [4096, 8192])
def test_square_full_coverage(n):
    A = synth.matrix(n, n, 2000 + n, 0)
    B = synth.matrix(n, n, 2000 + n, 1)
    full_size_check(to_dev(A), to_dev(B), A, B, (n, 1), n, n, n, 2000 + n, f"square {n}")



@pytest.mark.parametrize("M,N,K,variant,split", [(1024, 1024, 2048, "splitk", 4), (768, 768, 2048, "splitk", 4),
                                                 (1024, 1024, 4096, "splitk", 4), (1024, 1024, 1024, "main", 1),
                                                 (96, 8192, 8192, "splitk", 4), (200, 2048, 8192, "splitk", 8),
                                                 (256, 256, 16384, "splitk", 32), (128, 128, 65536, "splitk", 64)])
def test_auto_split_k_on_small_products(M, N, K, variant, split):
    # Split-K on the 128 x 128 LDS-DMA tile from K = 2048 while the 128 x
    # 128 tiles fill at most half the compute units: one workgroup per
    # compute unit, K ranges of at least 512 k.  Integer inputs keep every
    # sum exact, so the split plan gives the main plan's bits, and sampled
    # rows the oracle's.
    A = synth.matrix(M, K, 2700 + M, 0, "int")
    B = synth.matrix(K, N, 2700 + K, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (p["variant"], p["split_k"]) == (variant, split), p
    got = run(a, b, Out(M, N))
    assert_bits_equal(got, run(a, b, Out(M, N), variant="main"), f"{M}x{N}x{K} auto {p['variant']} vs main")
    rows = band_rows(M)
    assert_bits_equal(got[rows], reference(A, B, rows), f"{M}x{N}x{K} auto, sampled rows")

@pytest.mark.parametrize("M,N,K,tile", [(1024, 1024, 1024, 8), (768, 768, 768, 8),
                                        (1792, 1792, 1792, 7), (2048, 2048, 1024, 7),
                                        (2048, 2048, 2048, 7), (3072, 2048, 1024, 14),
                                        (2100, 2304, 2056, 14), (2100, 2300, 2056, 14),
                                        (1000, 4100, 2048, 1), (1000, 2052, 2048, 1)])
def test_main_tile_rule(M, N, K, tile):
    # The 64 x 128 LDS-DMA tile up to a quarter wave of 128 x 128 tiles, the
    # 128 x 128 LDS-DMA tile below 80 tiles of 256 x 256 (on 256 compute
    # units), the 256 x 256 tile from there on.  A B whose rows are not
    # 16-byte multiples (N = 2300, 4100) is packed for the big tile from M =
    # 1024 on; below that it keeps the 128 x 128 register tile, as does a B
    # with N % 8 != 0 in 16-byte rows (N = 2052).
    # Integer inputs keep every fp32 sum exact, so the automatic plan and the
    # other tile give the same bits, which sampled rows check against the
    # oracle (the first and last rows and one in every 256-row band).
    A = synth.matrix(M, K, 2500 + M, 0, "int")
    B = synth.matrix(K, N, 2500 + M, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (p["variant"], p["tile_id"]) == ("main", tile), p
    got = run(a, b)
    other = run(a, b, variant="main", tile=1 if p["tile_id"] != 1 else 14)
    assert_bits_equal(got, other, f"{M}x{N}x{K} tile {p['tile_id']} against the other tile")
    rows = band_rows(M)
    assert_bits_equal(got[rows], reference(A, B, rows), f"{M}x{N}x{K} sampled rows")


# ------------------------------------------------------------------ LDS-DMA tiles, K remainders

@pytest.mark.parametrize("tile", [7, 8, 13, 14])
@pytest.mark.parametrize("K", [32, 64, 96, 100, 160, 241])
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_dma_tiles_k_remainders(tile, K, b_layout):
    # Whole 64-k super-steps, an odd 32-k step and ragged K tails, on a tile
    # grid with ragged M and N edges; integer sums stay exact in fp32.
    M, N = 300, 264
    for mode in ("int", "uniform"):
        A = synth.matrix(M, K, 8000 + K, 0, mode)
        B = synth.matrix(K, N, 8000 + K, 1, mode)
        ref = reference(A, B)
        # Rows of A (and of a K-contiguous B) padded with NaN to a multiple of
        # 8 elements: every K tail is followed by poison that must never be read.
        pad = (-K) % 8 + 8
        a = place(A, "row", (1, pad))
        b = to_dev(B) if b_layout == "row" else place(B, "col", (1, pad))
        assert g.plan(a, b, variant="main", tile=tile)["tile_id"] == tile
        for kw in (dict(variant="main", tile=tile), dict(variant="splitk", tile=tile, split_k=3)):
            check(run(a, b, Out(M, N), **kw), ref, mode, f"dma tile K={K} {mode} {kw}")


@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_main_tile_edge_blocks(b_layout):
    # Last tile row / column of the 256x256 tile with every count of live
    # 32-wide blocks per wave (a wave owns 64 rows x 128 columns): rows past
    # M and columns past N are skipped by the edge tiles' MFMA predicate.
    K = 96
    for M in (257, 321, 449):
        for N in (264, 296, 352, 424, 488):
            A = synth.matrix(M, K, 8500 + M, 0, "int")
            B = synth.matrix(K, N, 8500 + N, 1, "int")
            ref = reference(A, B)
            a, b = to_dev(A), (to_dev(B) if b_layout == "row" else place(B, "col"))
            assert g.plan(a, b, variant="main", tile=14)["tile_id"] == 14
            for kw in (dict(variant="main", tile=14), dict(variant="splitk", tile=14, split_k=2)):
                check(run(a, b, Out(M, N), **kw), ref, "int", f"edge blocks {M}x{N} {kw}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_main_tile_output_store_forms(fmt):
    # The 256x256 tile writes C through LDS in whole 16-byte chunks when C is
    # 16-byte aligned with ldc % 8 == 0 and either the tile's columns lie
    # inside N or N % 8 == 0 (rows past M and chunks past N left out), and
    # element by element otherwise.  Each form, and their mix within one
    # call (N % 8 != 0: staged inner tiles, direct last tile column), against
    # the oracle, with NaN-filled outputs and canaries around them.
    # (N % 8 != 0 needs a K-contiguous B on this tile.)
    K = 64
    cases = [(300, 520, None, 64, "row"),    # staged, row and 8-column chunk edges
             (300, 520, 524, 64, "row"),     # ldc % 8 == 4: direct
             (300, 520, None, 65, "row"),    # C 2 bytes past a 16-byte boundary: direct
             (513, 300, None, 64, "col"),    # N % 8 == 4: staged inner, direct last column
             (512, 512, 520, 64, "row")]     # whole tiles, padded ldc: staged
    for M, N, ldc, guard, b_layout in cases:
        A = synth.matrix(M, K, 8700 + M, 0, "int", fmt=fmt)
        B = synth.matrix(K, N, 8700 + N, 1, "int", fmt=fmt)
        ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS,
                          dtype="bf16" if fmt == "bf16" else "f16")
        a, b = to_dev(A), place(B, b_layout)
        out = Out(M, N, ldc=ldc, guard=guard)
        if fmt == "bf16":
            a, b = a.view(torch.bfloat16), b.view(torch.bfloat16)
            out.view = out.view.view(torch.bfloat16)
        assert g.plan(a, b, out=out.view, variant="main", tile=14)["tile_id"] == 14
        got = run(a, b, out, variant="main", tile=14)
        assert_bits_equal(got, ref, f"{fmt} {M}x{N} ldc={ldc or N} guard={guard} B {b_layout}")


# ------------------------------------------------------------------ skinny / decode

@pytest.mark.parametrize("M", [1, 7, 16, 33, 64])
def test_skinny_full(M):
    N, K = 2048, 7168
    A = synth.matrix(M, K, 3000 + M, 0)
    B = synth.matrix(K, N, 3000 + M, 1)
    ref = reference(A, B)
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    assert p["variant"] == "skinny"
    for kw in (dict(variant="auto"), dict(variant="skinny", split_k=1),
               dict(variant="skinny", split_k=8), dict(variant="skinny", tile=3),
               dict(variant="main"), dict(variant="splitk", split_k=5)):
        check(run(a, b, Out(M, N), **kw), ref, "uniform", f"skinny M={M} {kw}")


@pytest.mark.parametrize("M", [1, 16, 64])
def test_skinny_integer_exact(M):
    N, K = 2048, 128
    A = synth.matrix(M, K, 3100 + M, 0, "int")
    B = synth.matrix(K, N, 3100 + M, 1, "int")
    ref = reference(A, B)
    a, b = to_dev(A), to_dev(B)
    for kw in (dict(variant="auto"), dict(variant="skinny", split_k=2)):
        check(run(a, b, Out(M, N), **kw), ref, "int", f"skinny int M={M} {kw}")


def test_split_k_512x512x65536():
    M = N = 512
    K = 65536
    A = synth.matrix(M, K, 3004, 0)
    B = synth.matrix(K, N, 3004, 1)
    a, b = to_dev(A), to_dev(B)
    p = full_size_check(a, b, A, B, (N, 1), M, N, K, 3004, "split-K 512x512x65536", points=20000,
                        band=64)
    assert p["variant"] == "splitk" and p["split_k"] > 1
    first = run(a, b)
    assert_bits_equal(run(a, b), first, "split-K rerun")
    rows = band_rows(M, 64)
    ref = reference(A, B, rows)
    for kw in (dict(variant="splitk", split_k=16), dict(variant="splitk", split_k=7),
               dict(variant="main")):
        check(run(a, b, **kw)[rows], ref, "uniform", f"split-K {kw}")


# ------------------------------------------------------------------ full-size configurations

def test_moe_131072x2048x7168_full_coverage():
    M, N, K = 131072, 2048, 7168
    A = synth.matrix(M, K, 4001, 0)
    B = synth.matrix(K, N, 4001, 1)
    a, b = to_dev(A), to_dev(B)
    p = full_size_check(a, b, A, B, (N, 1), M, N, K, 4001, "MoE 131072x2048x7168")
    assert p["variant"] == "main"


def test_int64_stride_262181x1061x8192_full_coverage():
    M, N, K = 262181, 1061, 8192
    A = synth.matrix(M, K, 5001, 0)
    Bt = synth.matrix(K, N, 5001, 1, order="col")     # stored [N][K]
    a = to_dev(A)
    b = to_dev(Bt).t()                                  # [K, N] view, strides (1, K)
    assert b.stride() == (1, K)
    rows = band_rows(M)
    assert rows.max() >= 262144 and (rows >= 131072).sum() > 500   # offsets past 2^31 elements
    full_size_check(a, b, A, Bt, (1, K), M, N, K, 5001, "262181x1061x8192")


def test_int64_stride_integer_slice_exact():
    """K = 128 slice of the stress buffers: element offsets past 2^31 are
    checked bit-exactly (the buffers are NaN outside the slice)."""
    M, N, Kfull, K = 262181, 1061, 8192, 128
    A = synth.matrix(M, K, 5002, 0, "int")
    Bt = synth.matrix(K, N, 5002, 1, "int", order="col")   # [N][K]
    abuf = torch.full((M, Kfull), float("nan"), dtype=torch.float16, device=DEV)
    abuf[:, :K].copy_(to_dev(A))
    bbuf = torch.full((N, Kfull), float("nan"), dtype=torch.float16, device=DEV)
    bbuf[:, :K].copy_(to_dev(Bt))
    a = abuf[:, :K]
    b = bbuf[:, :K].t()
    assert a.stride() == (Kfull, 1) and b.stride() == (1, Kfull)
    rows = np.array([0, 1, 131071, 131072, 262143, 262144, 262145, M - 1])
    ref = reference(A, np.ascontiguousarray(Bt.T), rows)
    for kw in (dict(variant="auto"), dict(variant="splitk", split_k=2),
               dict(variant="streamk", split_k=2)):
        gpu = run(a, b, **kw)
        check(gpu[rows], ref, "int", f"int64 slice {kw}")


def test_offsets_of_2_pow_32_elements():
    """Row, k and output strides of exactly 2^32 elements: a 32-bit offset
    would wrap to 0 and read or write the wrong element (Triton article,
    section "addresses and bounds in one short kernel")."""
    big = 2 ** 32
    N = 64
    # lda_m = 2^32
    buf = dev_nan(big + 8)
    buf[0] = 1.0
    buf[big] = 2.0
    a = torch.as_strided(buf, (2, 1), (big, 1))
    B = synth.matrix(1, N, 5003, 1, "int")
    ref = reference(np.array([[0x3C00], [0x4000]], np.uint16), B)
    check(run(a, to_dev(B)), ref, "int", "lda_m = 2^32")
    del buf, a
    # ldb_k = 2^32
    bbuf = dev_nan(big + N + 8)
    B2 = synth.matrix(2, N, 5004, 1, "int")
    bbuf[:N].copy_(to_dev(B2[0]))
    bbuf[big:big + N].copy_(to_dev(B2[1]))
    b = torch.as_strided(bbuf, (2, N), (big, 1))
    A2 = synth.matrix(4, 2, 5004, 0, "int")
    check(run(to_dev(A2), b), reference(A2, B2), "int", "ldb_k = 2^32")
    del bbuf, b
    # ldc = 2^32
    cbuf = torch.full((big + N + 8,), 7.0, dtype=torch.float16, device=DEV)
    c = torch.as_strided(cbuf, (2, N), (big, 1))
    A3 = synth.matrix(2, 3, 5005, 0, "int")
    B3 = synth.matrix(3, N, 5005, 1, "int")
    say("gemm ldc = 2^32")
    g.gemm(to_dev(A3), to_dev(B3), out=c)
    torch.cuda.synchronize()
    ref = reference(A3, B3)
    got = np.stack([to_host(cbuf[:N]), to_host(cbuf[big:big + N])])
    assert_bits_equal(got, ref, "ldc = 2^32")
    assert torch.all(cbuf[N:N + 8] == 7.0) and torch.all(cbuf[big - 8:big] == 7.0)


def _rows_at(bits, ld):
    """fp16 bits [R, C] into a NaN buffer with row stride ld (elements)."""
    R, C = bits.shape
    buf = dev_nan((R - 1) * ld + C + 8)
    v = torch.as_strided(buf, (R, C), (ld, 1))
    v.copy_(to_dev(bits))
    return buf, v


@pytest.mark.parametrize("which", ["A", "B_n", "B_k"])
def test_dma_tile_stride_limit(which):
    """The 256x256 LDS-DMA tile addresses its operands with 32-bit lane
    offsets over 256 rows: at a row stride of 2^23 elements (lane offsets up
    to 255 * 2^24 bytes, just under 2^32) it still runs, with the last tile
    row clamped; one step past the limit the plan hands over to another
    tile.  Integer inputs, bit-exact against the oracle."""
    M, N, K = 257, 264, 96
    A = synth.matrix(M, K, 16000, 0, "int")
    B = synth.matrix(K, N, 16001, 1, "int")
    ref = reference(A, B)
    lim = 1 << 23
    for ld, dma in ((lim, True), (lim + 8, False)):
        if which == "A":
            buf, a = _rows_at(A, ld)
            b = to_dev(B)
        elif which == "B_n":           # N-contiguous B, k-rows ld apart
            buf, b = _rows_at(B, ld)
            a = to_dev(A)
        else:                          # K-contiguous B stored [N, K], n-rows ld apart
            buf, bt = _rows_at(np.ascontiguousarray(B.T), ld)
            b = bt.t()
            a = to_dev(A)
        kw = dict(variant="main", tile=14)
        p = g.plan(a, b, **kw)
        assert (p["tile_id"] == 14) == dma, (which, ld, p)
        check(run(a, b, **kw), ref, "int", f"{which} stride {ld} plan {p}")
        del buf, a, b
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ properties

def test_repeat_runs_are_bit_identical():
    M, N, K = 700, 600, 3000
    A = synth.matrix(M, K, 6001, 0)
    B = synth.matrix(K, N, 6001, 1)
    a, b = to_dev(A), to_dev(B)
    for kw in VARIANTS:
        first = run(a, b, **kw)
        assert_bits_equal(run(a, b, **kw), first, f"rerun {kw}")


def test_split_counts_agree_on_integers():
    M, N, K = 200, 300, 128
    A = synth.matrix(M, K, 6002, 0, "int")
    B = synth.matrix(K, N, 6002, 1, "int")
    a, b = to_dev(A), to_dev(B)
    base = run(a, b, variant="main")
    assert_bits_equal(base, reference(A, B), "main")
    for s in (1, 2, 3, 7, 16):
        assert_bits_equal(run(a, b, variant="splitk", split_k=s), base, f"split {s}")


def test_caller_workspace_is_used_and_needs_no_reset():
    M, N, K = 512, 512, 8192
    A = synth.matrix(M, K, 6003, 0)
    B = synth.matrix(K, N, 6003, 1)
    a, b = to_dev(A), to_dev(B)
    need = g.workspace_bytes(M, N, K, variant="splitk", split_k=8)
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device=DEV)
    first = run(a, b, workspace=ws, variant="splitk", split_k=8)
    ws.fill_(12345.0)
    assert_bits_equal(run(a, b, workspace=ws, variant="splitk", split_k=8), first, "workspace")
    rows = np.array([0, 255, 511])
    check(first[rows], reference(A, B, rows), "uniform", "workspace")
    with pytest.raises(g.GemmError) as e:
        g.gemm(a, b, workspace=ws[:16], variant="splitk", split_k=8)
    assert e.value.status == -6


# ------------------------------------------------------------------ decode kernel (M <= 64, N-contiguous B)

def _decode_case(M, N, K, mode, ldb_pad=0, split=0, seed=7000, b_layout="row"):
    # b_layout "row": B [K, N] N-contiguous (rows padded by ldb_pad);
    # "col": B as [N, K] rows, each padded to a multiple of 8 elements with at
    # least 8 NaN past K, so a read beyond K turns outputs into NaN.
    A = synth.matrix(M, K, seed + M, 0, mode)
    B = synth.matrix(K, N, seed + N, 1, mode)
    ref = reference(A, B)
    a = place(A, "row", (1, 8))
    if b_layout == "col":
        b = place(B, "col", (1, (-K) % 8 + 8))
    else:
        b = place(B, "row", (0, ldb_pad)) if ldb_pad else to_dev(B)
    p = g.plan(a, b, variant="skinny", split_k=split)
    assert p["b_path"] == ("kvec" if b_layout == "col" else "rvec") and p["tile_n"] == 128 and \
        p["tile_m"] == (16 if M <= 16 else 32 if M <= 32 else 64), p
    need = p["workspace_bytes"]
    ws = torch.full((max(need, 4096) // 4 + 64,), float("nan"), dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(2):
        outs.append(run(a, b, Out(M, N), workspace=ws, variant="skinny", split_k=split))
        ws.fill_(-7.0)                       # the workspace needs no initialisation
    assert_bits_equal(outs[1], outs[0], f"decode rerun M={M} N={N} K={K} B {b_layout}")
    check(outs[0], ref, mode, f"decode M={M} N={N} K={K} pad={ldb_pad} split={split} B {b_layout}")
    return p


DECODE_CASES = [(M, "row") for M in (1, 2, 3, 4, 16, 17, 40, 64)] + [(M, "col") for M in (1, 2, 3, 4, 16)]


@pytest.mark.parametrize("M,b_layout", DECODE_CASES)
def test_decode_kernel_uniform(M, b_layout):
    p = _decode_case(M, 2048, 7168, "uniform", b_layout=b_layout)
    assert p["split_k"] > 1
    _decode_case(M, 1001, 300, "uniform", ldb_pad=7, b_layout=b_layout)   # ragged last vector and last split
    _decode_case(M, 520, 1024, "uniform", split=1, b_layout=b_layout)     # one split: direct store
    _decode_case(M, 264, 2500, "uniform", split=2, b_layout=b_layout)     # K ranges longer than one A chunk
    _decode_case(M, 1001, 7168, "uniform", ldb_pad=7, b_layout=b_layout)  # 16-lane reduction, ragged N
    if b_layout == "col":
        _decode_case(M, 130, 301, "uniform", b_layout=b_layout)         # K tail inside a k-octet


@pytest.mark.parametrize("M,b_layout", [(M, "row") for M in (1, 3, 4, 16, 33, 64)] +
                         [(M, "col") for M in (1, 3, 4, 16)])
def test_decode_kernel_integer_exact(M, b_layout):
    for split in (0, 1, 3):
        _decode_case(M, 777, 128, "int", ldb_pad=7, split=split, b_layout=b_layout)
        _decode_case(M, 2048, 128, "int", split=split, b_layout=b_layout)
        _decode_case(M, 2048, 130, "int", split=split, b_layout=b_layout)   # A rows not 16-byte aligned
        if b_layout == "col":
            _decode_case(M, 300, 133, "int", split=split, b_layout=b_layout)


def test_skinny_plans_by_b_layout():
    # K-contiguous B: the decode kernel (128-column strips) up to 16 rows of
    # A, the skinny MFMA tiles from 17 to 64 rows; N-contiguous B: the decode
    # kernel up to 64 rows.
    K, N = 7168, 2048
    for M, tile_m, decode in ((1, 16, True), (16, 16, True), (17, 32, False), (64, 64, False)):
        a = to_dev(synth.matrix(M, K, 1, 0))
        p = g.plan(a, place(synth.matrix(K, N, 1, 1), "col"))
        assert (p["variant"], p["b_path"], p["tile_m"]) == ("skinny", "kvec", tile_m), p
        assert (p["tile_n"] == 128) == decode, p
        q = g.plan(a, to_dev(synth.matrix(K, N, 1, 1)))
        assert (q["variant"], q["b_path"], q["tile_n"]) == ("skinny", "rvec", 128), q


def test_wrapper_rejects_bad_arguments():
    a = torch.zeros((4, 8), dtype=torch.float16, device=DEV)
    b = torch.zeros((8, 3), dtype=torch.float16, device=DEV)
    with pytest.raises(TypeError):
        g.gemm(a.float(), b)
    with pytest.raises(ValueError):
        g.gemm(a, b.t())
    with pytest.raises(ValueError):
        g.gemm(a[:0], b)
    with pytest.raises(ValueError):
        g.gemm(a.cpu(), b)
    big = torch.zeros(64, dtype=torch.float16, device=DEV)
    with pytest.raises(g.GemmError) as e:                  # output overlapping an input
        g.gemm(big[:32].view(4, 8), b, out=big[16:28].view(4, 3))
    assert e.value.status == -5
