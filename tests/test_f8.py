"""GPU parity of the FP8 entry points (gemm_f8*, TileLang tutorial ch. 14,
section 5): OCP E4M3 / E5M2 operands, fp32 accumulation, binary16 output,
against the oracle's FP8 product on the same seeded inputs; B given as
[N, K] rows (K-contiguous) and as [K, N] rows (N-contiguous).  Acceptance as
for fp16: bit-exact on integer inputs (exact in both FP8 formats, sums exact
in fp32), the elementwise tolerance 1e-2 + 2e-3 |C| on U(-1, 1) inputs
rounded to FP8.  Operand rows are padded with the NaN byte 0x7F (NaN in both
formats), which must never reach an output.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, ORACLE_THREADS, Out, assert_bits_equal, assert_close, full_size_check,
                      say, to_host)

pytestmark = pytest.mark.gpu

TORCH_F8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


def f8_rows(bits, fmt, pad=None):
    """uint8 [R, K] -> FP8 device view [R, K] whose rows are padded to a
    multiple of 16 bytes (at least 16 more) with 0x7F."""
    R, K = bits.shape
    pad = (-K) % 16 + 16 if pad is None else pad
    buf = np.full((R, K + pad), 0x7F, dtype=np.uint8)
    buf[:, :K] = bits
    return torch.from_numpy(buf).to(DEV).view(TORCH_F8[fmt])[:, :K]


def inputs(M, N, K, seed, mode, fa, fb):
    A = synth.matrix(M, K, seed, 0, mode, fmt=fa)
    Bt = synth.matrix(K, N, seed, 1, mode, fmt=fb, order="col")    # stored [N][K]
    return A, Bt


def reference(A, Bt, fa, fb, rows=None):
    K = A.shape[1]
    B = np.ascontiguousarray(Bt.T)
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (B.shape[1], 1), A.shape[0], B.shape[1], K, dtype="f8",
                       fmt_a=fa, fmt_b=fb, nthreads=ORACLE_THREADS)


def run(a, b, out, **kw):
    say(f"gemm_f8 M={a.shape[0]} N={b.shape[1]} K={a.shape[1]} {a.dtype}/{b.dtype} "
        f"a.stride={a.stride()} b.stride={b.stride()} opts={kw}")
    g.gemm(a, b, out=out.view, **kw)
    torch.cuda.synchronize()
    return out.result()


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_f8_parity_ragged(fa, fb, mode):
    M, N, K = 600, 520, 700
    A, Bt = inputs(M, N, K, 14000, mode, fa, fb)
    ref = reference(A, Bt, fa, fb)
    a, b = f8_rows(A, fa), f8_rows(Bt, fb).t()
    for kw in (dict(variant="main"), dict(variant="splitk", split_k=3),
               dict(variant="streamk", split_k=2)):
        got = run(a, b, Out(M, N), **kw)
        what = f"f8 {fa}x{fb} {mode} {kw}"
        if mode == "int":
            assert_bits_equal(got, ref, what)
        else:
            assert_close(got, ref, what)


def test_f8_output_store_forms():
    # As for the 16-bit tile: C staged through LDS in 16-byte chunks (16-byte
    # aligned C, ldc % 8 == 0, tile columns inside N or N % 8 == 0), element
    # by element otherwise, and both within one call when N % 8 != 0.
    K = 256
    for M, N, ldc, guard in ((300, 520, None, 64), (300, 520, 524, 64), (300, 520, None, 65),
                             (513, 300, None, 64)):
        A, Bt = inputs(M, N, K, 14050 + M + N, "int", "e4m3", "e4m3")
        got = run(f8_rows(A, "e4m3"), f8_rows(Bt, "e4m3").t(), Out(M, N, ldc=ldc, guard=guard),
                  variant="main")
        assert_bits_equal(got, reference(A, Bt, "e4m3", "e4m3"),
                          f"f8 {M}x{N} ldc={ldc or N} guard={guard}")


@pytest.mark.parametrize("K", [1, 33, 64, 100, 128, 192, 255, 384])
def test_f8_k_tails(K):
    # Whole 128-k super-steps, an odd 64-k step and ragged tails, byte by byte.
    M, N = 300, 264
    A, Bt = inputs(M, N, K, 14100 + K, "int", "e4m3", "e4m3")
    ref = reference(A, Bt, "e4m3", "e4m3")
    got = run(f8_rows(A, "e4m3"), f8_rows(Bt, "e4m3").t(), Out(M, N), variant="main")
    assert_bits_equal(got, ref, f"f8 K={K}")


def test_f8_edge_blocks():
    # Last tile row / column with every count of live 32-wide blocks.
    K = 192
    for M in (257, 321, 449):
        for N in (264, 296, 352, 424, 488):
            A, Bt = inputs(M, N, K, 14200 + M + N, "int", "e5m2", "e4m3")
            ref = reference(A, Bt, "e5m2", "e4m3")
            got = run(f8_rows(A, "e5m2"), f8_rows(Bt, "e4m3").t(), Out(M, N), variant="main")
            assert_bits_equal(got, ref, f"f8 edge blocks {M}x{N}")


def test_f8_moe_shape_full_coverage():
    # The 131072 x 2048 x 7168 product with E4M3 operands (B as [N, K]
    # weights) on its automatic (packing) plan: every output written, one
    # oracle row per 256-row band and 10^5 oracle points over the output.
    M, N, K = 131072, 2048, 7168
    say("f8 MoE: generating inputs")
    A, Bt = inputs(M, N, K, 14300, "uniform", "e4m3", "e4m3")
    a = torch.from_numpy(A).to(DEV).view(torch.float8_e4m3fn)
    b = torch.from_numpy(Bt).to(DEV).view(torch.float8_e4m3fn).t()
    p = full_size_check(a, b, A, Bt, (1, K), M, N, K, 14300, "f8 MoE", dtype="f8")
    assert p["tile_id"] == 15 and p["b_path"] == "packed", p     # the packing plan


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_f8_auto_packs_kcontig_b(fa, fb):
    # M past the packing threshold, ragged M, N and K (700 = 5 x 128 + 60):
    # B packed as byte pairs, then the packed-B FP8 kernel; same bits as the
    # oracle and as the direct plan.
    M, N, K = 16384 + 37, 300, 700
    A, Bt = inputs(M, N, K, 14400, "int", fa, fb)
    ref = reference(A, Bt, fa, fb)
    a, b = f8_rows(A, fa), f8_rows(Bt, fb).t()
    p = g.plan(a, b)
    assert p["b_path"] == "packed" and p["tile_id"] == 15, p
    assert p["workspace_bytes"] == g.lib.gemm_f16_packed_b_bytes(K // 2, N), p
    assert_bits_equal(run(a, b, Out(M, N)), ref, f"f8 packing plan {fa}x{fb}")
    assert g.plan(a, b, variant="main")["b_path"] == "kvec"
    assert_bits_equal(run(a, b, Out(M, N), variant="main"), ref, f"f8 direct plan {fa}x{fb}")


def test_f8_auto_pack_streamk():
    # 325 tiles: a stream-K tail of 69; the packed FP8 B in front of the
    # partials, against the same split forced without packing.
    M, N, K = 16384 + 37, 1061, 2100
    A, Bt = inputs(M, N, K, 14900, "int", "e4m3", "e4m3")
    a, b = f8_rows(A, "e4m3"), f8_rows(Bt, "e4m3").t()
    p = g.plan(a, b)
    if p["variant"] != "streamk":
        pytest.skip(f"this device's compute-unit count gives no stream-K tail here: {p}")
    assert p["b_path"] == "packed", p
    got = run(a, b, Out(M, N))
    direct = run(a, b, Out(M, N), variant="streamk", split_k=p["split_k"])
    assert_bits_equal(got, direct, "f8 stream-K packed vs direct")
    rng = np.random.default_rng(14900)
    rows = np.unique(np.concatenate([[0, 255, 16383, 16384, M - 1], rng.integers(0, M, 8)]))
    assert_bits_equal(got[rows], reference(A, Bt, "e4m3", "e4m3", rows), "f8 stream-K sampled rows")


def test_f8_odd_k_packed_bytewise():
    # K odd: the byte-pair packing cannot zero the byte past K, so B packs
    # byte by byte; 701 = 5 x 128 + 61.
    M, N, K = 16384, 264, 701
    A, Bt = inputs(M, N, K, 14500, "int", "e4m3", "e4m3")
    a, b = f8_rows(A, "e4m3"), f8_rows(Bt, "e4m3").t()
    p = g.plan(a, b)
    assert p["b_path"] == "packed" and p["workspace_bytes"] == g.lib.gemm_f16_packed_b_bytes(351, N), p
    assert_bits_equal(run(a, b, Out(M, N)), reference(A, Bt, "e4m3", "e4m3"), "f8 odd K")


def test_f8_stride_limit():
    # A rows 2^24 bytes apart, the largest stride the FP8 tile takes: lane
    # offsets of the DMA reach 255 * 2^24 bytes, just under 2^32; the last
    # tile row is clamped (M = 257).  Integer inputs, bit-exact.
    M, N, K = 257, 264, 192
    A, Bt = inputs(M, N, K, 14400, "int", "e4m3", "e4m3")
    ref = reference(A, Bt, "e4m3", "e4m3")
    ld = 1 << 24
    buf = torch.full(((M - 1) * ld + K + 16,), 0x7F, dtype=torch.uint8, device=DEV)
    a8 = torch.as_strided(buf, (M, K), (ld, 1))
    a8.copy_(torch.from_numpy(A).to(DEV))
    a = a8.view(torch.float8_e4m3fn)
    b = f8_rows(Bt, "e4m3").t()
    got = run(a, b, Out(M, N), variant="main")
    assert_bits_equal(got, ref, "f8 lda_m = 2^24")


# ---------------------------------------------------------------- N-contiguous B

def f8_krows(bits, fmt, pad=None):
    """uint8 B [K, N] -> FP8 device view [K, N] whose k-rows are padded to a
    multiple of 16 bytes (at least 16 more) with 0x7F (NaN)."""
    K, N = bits.shape
    pad = (-N) % 16 + 16 if pad is None else pad
    buf = np.full((K, N + pad), 0x7F, dtype=np.uint8)
    buf[:, :N] = bits
    return torch.from_numpy(buf).to(DEV).view(TORCH_F8[fmt])[:, :N]


def inputs_bn(M, N, K, seed, mode, fa, fb):
    A = synth.matrix(M, K, seed, 0, mode, fmt=fa)
    B = synth.matrix(K, N, seed, 1, mode, fmt=fb)        # [K, N] row-major
    return A, B


def reference_bn(A, B, fa, fb, rows=None):
    K, N = B.shape
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (N, 1), A.shape[0], N, K, dtype="f8", fmt_a=fa, fmt_b=fb,
                       nthreads=ORACLE_THREADS)


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_f8_bn_parity_ragged(fa, fb, mode):
    M, N, K = 600, 528, 700
    A, B = inputs_bn(M, N, K, 14500, mode, fa, fb)
    ref = reference_bn(A, B, fa, fb)
    a, b = f8_rows(A, fa), f8_krows(B, fb)
    assert b.stride(1) == 1
    for kw in (dict(variant="main"), dict(variant="splitk", split_k=3),
               dict(variant="streamk", split_k=2)):
        p = g.plan(a, b, **kw)
        assert p["b_path"] == "rvec" and p["tile_id"] == 15, p
        got = run(a, b, Out(M, N), **kw)
        what = f"f8 B [K, N] {fa}x{fb} {mode} {kw}"
        if mode == "int":
            assert_bits_equal(got, ref, what)
        else:
            assert_close(got, ref, what)


@pytest.mark.parametrize("fa,fb,K", [("e4m3", "e5m2", 700), ("e5m2", "e5m2", 333)])
def test_f8_bn_large_m_direct(fa, fb, K):
    # B [K, N] row-major past the packing threshold stays on the direct
    # N-major path (as fast as packed stages); ragged M, N and K.
    M, N = 16384 + 37, 304
    A, B = inputs_bn(M, N, K, 14800 + K, "int", fa, fb)
    a, b = f8_rows(A, fa), f8_krows(B, fb)
    p = g.plan(a, b)
    assert p["b_path"] == "rvec" and p["tile_id"] == 15 and p["workspace_bytes"] == 0, p
    assert_bits_equal(run(a, b, Out(M, N)), reference_bn(A, B, fa, fb), f"f8 B [K, N] {fa}x{fb} K={K}")


@pytest.mark.parametrize("K", [1, 7, 64, 100, 128, 192, 255, 384])
def test_f8_bn_k_tails(K):
    # Whole 128-k super-steps, an odd 64-k step and ragged tails (k-rows
    # past K are zero in the stage), byte by byte.
    M, N = 300, 272
    A, B = inputs_bn(M, N, K, 14600 + K, "int", "e4m3", "e5m2")
    ref = reference_bn(A, B, "e4m3", "e5m2")
    got = run(f8_rows(A, "e4m3"), f8_krows(B, "e5m2"), Out(M, N), variant="main")
    assert_bits_equal(got, ref, f"f8 B [K, N] K={K}")


def test_f8_bn_edge_blocks():
    # Last tile column with 1..7 live 32-wide blocks and half blocks (N a
    # multiple of 16), last tile row with every count of live 32-row blocks.
    K = 192
    for M in (257, 321, 449):
        for N in (16, 272, 304, 352, 432, 496):
            A, B = inputs_bn(M, N, K, 14700 + M + N, "int", "e4m3", "e4m3")
            ref = reference_bn(A, B, "e4m3", "e4m3")
            got = run(f8_rows(A, "e4m3"), f8_krows(B, "e4m3", pad=16 + 16 * (N % 32 == 0)),
                      Out(M, N), variant="main")
            assert_bits_equal(got, ref, f"f8 B [K, N] edge blocks {M}x{N}")


def test_f8_bn_moe_shape_full_coverage():
    # The 131072 x 2048 x 7168 product with E4M3 operands and B [K, N]
    # row-major, as the fp16 workload lays it out; checked as above.
    M, N, K = 131072, 2048, 7168
    say("f8 B [K, N] MoE: generating inputs")
    A, B = inputs_bn(M, N, K, 14800, "uniform", "e4m3", "e4m3")
    a = torch.from_numpy(A).to(DEV).view(torch.float8_e4m3fn)
    b = torch.from_numpy(B).to(DEV).view(torch.float8_e4m3fn)
    p = full_size_check(a, b, A, B, (N, 1), M, N, K, 14800, "f8 B [K, N] MoE", dtype="f8")
    assert p["tile_id"] == 15 and p["b_path"] == "rvec", p


F8_DECODE_CASES = [(1, 2048, 7168, {}), (16, 1040, 1000, {}), (17, 272, 130, {}),
                   (64, 528, 96, dict(variant="skinny")), (2, 16, 1, {}), (7, 48, 7, {}),
                   (3, 2048, 7168, dict(variant="skinny", split_k=1)),
                   (40, 1040, 2500, dict(variant="skinny", split_k=5))]


F8_DECODE_NK_CASES = [(1, 2048, 7168, {}), (16, 1030, 1000, {}), (5, 272, 130, {}), (1, 3, 1, {}),
                      (16, 1, 9, {}),
                      (3, 2048, 7168, dict(variant="skinny", split_k=1)),
                      (9, 1040, 2500, dict(variant="skinny", split_k=5))]


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_f8_decode(fa, fb, mode, b_layout):
    # Up to 32 rows of A with B as [K, N] rows (64 when forced), up to 16
    # with B as [N, K] rows: the decode kernel, the FP8 bytes widened to
    # binary16 (exact for both formats), fp32 sums over K ranges and the
    # fixed-order reduction.  The cases cover ragged last column strips (N =
    # 1040: 16 columns past the eighth strip; N = 1030 with [N, K] rows),
    # ragged last K ranges, 16, 32 and 64-row kernels, one K range (C
    # written directly) and forced splits; rows padded with NaN bytes past K
    # and N.
    for M, N, K, kw in (F8_DECODE_CASES if b_layout == "kn" else F8_DECODE_NK_CASES):
        A, Bt = inputs(M, N, K, 14400 + M + K, mode, fa, fb)
        ref = reference(A, Bt, fa, fb)
        a = f8_rows(A, fa)
        if b_layout == "kn":
            b = f8_rows(np.ascontiguousarray(Bt.T), fb)      # [K, N] rows
        else:
            b = f8_rows(Bt, fb).t()                          # [N, K] rows
        p = g.plan(a, b, **kw)
        assert p["variant"] == "skinny" and p["tile_n"] == 128, p
        if "split_k" in kw:
            assert p["split_k"] == kw["split_k"], p
        got = run(a, b, Out(M, N), **kw)
        what = f"f8 decode {fa}x{fb} {mode} {M}x{N}x{K} {kw} plan {p}"
        if mode == "int":
            assert_bits_equal(got, ref, what)
        else:
            assert_close(got, ref, what)


def test_f8_decode_plan_bounds():
    # The tiled plans (split over K) from 17 rows of A with B as [N, K] rows
    # and from 33 rows with B as [K, N] rows.
    for M, nk in ((17, True), (33, False)):
        N, K = 512, 4096
        A, Bt = inputs(M, N, K, 14480 + M, "int", "e4m3", "e4m3")
        a = f8_rows(A, "e4m3")
        b = f8_rows(Bt, "e4m3").t() if nk else f8_rows(np.ascontiguousarray(Bt.T), "e4m3")
        p = g.plan(a, b)
        assert p["variant"] != "skinny" and p["tile_id"] in (7, 15), p
        assert_bits_equal(run(a, b, Out(M, N)), reference(A, Bt, "e4m3", "e4m3"), f"f8 M = {M}, nk {nk}")
    A, Bt = inputs(32, 512, 4096, 14532, "int", "e4m3", "e4m3")
    assert g.plan(f8_rows(A, "e4m3"), f8_rows(np.ascontiguousarray(Bt.T), "e4m3"))["variant"] == "skinny"
    A, Bt = inputs(16, 512, 4096, 14548, "int", "e4m3", "e4m3")
    assert g.plan(f8_rows(A, "e4m3"), f8_rows(Bt, "e4m3").t())["variant"] == "skinny"


@pytest.mark.parametrize("tile", [7, 8])
@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_f8_128_wide_dma_tiles(tile, fa, fb, mode):
    # FP8 with B as [N, K] rows on the 128 x 128 and 64 x 128 LDS-DMA tiles:
    # byte pairs through the 16-bit stages (64 k per stage) and one f8f6f4
    # MFMA per block and stage; ragged M, N and K tails, rows padded with NaN
    # bytes; main and split-K.
    M, N, K = 600, 520, 700
    A, Bt = inputs(M, N, K, 14600 + tile, mode, fa, fb)
    ref = reference(A, Bt, fa, fb)
    a, b = f8_rows(A, fa), f8_rows(Bt, fb).t()
    for kw in (dict(variant="main", tile=tile), dict(variant="splitk", tile=tile, split_k=3)):
        p = g.plan(a, b, **kw)
        assert p["tile_id"] == tile, p
        got = run(a, b, Out(M, N), **kw)
        what = f"f8 tile {tile} {fa}x{fb} {mode} {kw}"
        if mode == "int":
            assert_bits_equal(got, ref, what)
        else:
            assert_close(got, ref, what)


@pytest.mark.parametrize("K", [2, 64, 100, 128, 130, 254, 1000])
def test_f8_128_wide_dma_tiles_k_tails(K):
    M, N = 300, 264
    A, Bt = inputs(M, N, K, 14700 + K, "int", "e5m2", "e4m3")
    ref = reference(A, Bt, "e5m2", "e4m3")
    a, b = f8_rows(A, "e5m2"), f8_rows(Bt, "e4m3").t()
    for tile in (7, 8):
        assert_bits_equal(run(a, b, Out(M, N), variant="main", tile=tile), ref, f"f8 tile {tile} K={K}")


def test_f8_odd_k_hands_the_128_wide_tiles_over():
    # Byte pairs need K even: an odd K, or B as [K, N] rows, runs on the FP8 tile.
    M, N, K = 300, 272, 129
    A, Bt = inputs(M, N, K, 14790, "int", "e4m3", "e4m3")
    a = f8_rows(A, "e4m3")
    for b in (f8_rows(Bt, "e4m3").t(), f8_rows(np.ascontiguousarray(Bt.T), "e4m3")):
        p = g.plan(a, b, variant="main", tile=7)
        assert p["tile_id"] == 15, p
        assert_bits_equal(run(a, b, Out(M, N), variant="main", tile=7), reference(A, Bt, "e4m3", "e4m3"),
                          f"f8 tile 7 handed over, b.stride={b.stride()}")


@pytest.mark.parametrize("M,N,K,b_layout,variant,tile", [
    (1024, 1024, 1024, "nk", "main", 8), (2048, 2048, 2048, "nk", "main", 7),
    (3072, 3072, 3072, "nk", "main", 15), (1024, 1024, 2048, "nk", "main", 8),
    (1024, 1024, 8192, "nk", "splitk", 7), (2048, 2048, 2048, "kn", "main", 15),
    (2048, 2048, 2049, "nk", "main", 15), (32, 2048, 7168, "nk", "splitk", 7),
    (48, 2048, 7168, "kn", "splitk", 15)])
def test_f8_tile_rule(M, N, K, b_layout, variant, tile):
    # FP8 with B as [N, K] rows and K even takes the fp16 rule's 128-wide
    # LDS-DMA tiles below 80 tiles of 256 x 256 (256 compute units), split K
    # from K >= 4096; other layouts and larger grids take the
    # FP8 tile.  Integer inputs: every plan gives the oracle's bits on
    # sampled rows.
    A, Bt = inputs(M, N, K, 14800 + M + K, "int", "e4m3", "e4m3")
    a = f8_rows(A, "e4m3")
    b = f8_rows(Bt, "e4m3").t() if b_layout == "nk" else f8_rows(np.ascontiguousarray(Bt.T), "e4m3")
    p = g.plan(a, b)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (p["variant"], p["tile_id"]) == (variant, tile), p
    got = run(a, b, Out(M, N))
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(7, M, 97)]))
    assert_bits_equal(got[rows], reference(A, Bt, "e4m3", "e4m3", rows), f"f8 {M}x{N}x{K} {b_layout} plan {p}")
