"""The automatic plan's dispatch rules on the CPU, through
gemm_f16_plan_cus (the plan for a device with a given compute-unit count,
with no device query).  Every expected choice below is the one the GPU
timings of the rule picked; the GPU parity tests run the same shapes.
Pointers are aligned stand-in addresses: planning reads their alignment
only."""
import ctypes

import pytest

import dense_tiled_gemm_fp16_amd as g
from dense_tiled_gemm_fp16_amd import _lib

PA, PB, PC = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000
MAIN, SKINNY, SPLITK, STREAMK = 1, 2, 3, 5
GATHER, KVEC, RVEC, PACKED = 0, 1, 2, 3
T128, T128_DMA, T64_DMA, T256_DMA = 1, 7, 8, 14


def plan(M, N, K, lda=None, ldb=None, a="row", b="row", cus=256, A=PA, B=PB, opts=None):
    """A [M, K]: "row" (row stride lda, default K), "mc" (M-contiguous,
    column stride lda, default M) or "strided" (every other column).
    B [K, N]: "row" (row stride ldb, default N) or "nk" (B as [N, K] rows,
    row stride ldb, default K)."""
    if a == "row":
        lda_m, lda_k = (lda or K), 1
    elif a == "mc":
        lda_m, lda_k = 1, (lda or M)
    else:
        lda_m, lda_k = 2 * K, 2
    ldb_k, ldb_n = ((ldb or N), 1) if b == "row" else (1, (ldb or K))
    info = _lib.PlanInfo()
    rc = g.lib.gemm_f16_plan_cus(A, lda_m, lda_k, B, ldb_k, ldb_n, PC, N, M, N, K, cus,
                                 ctypes.byref(opts) if opts else None, ctypes.byref(info))
    assert rc == 0, rc
    return info


def test_compute_unit_count_is_checked():
    info = _lib.PlanInfo()
    for cus in (0, -1, 65537):
        assert g.lib.gemm_f16_plan_cus(PA, 64, 1, PB, 64, 1, PC, 64, 64, 64, 64, cus, None,
                                       ctypes.byref(info)) == -7


@pytest.mark.parametrize("M,N,K,tile", [(2048, 2048, 2048, T128_DMA), (2304, 2304, 2304, T256_DMA),
                                        (3072, 2048, 1024, T256_DMA), (2048, 2048, 1024, T128_DMA),
                                        (1792, 1792, 1792, T128_DMA), (1536, 1536, 1536, T128_DMA),
                                        (1024, 1024, 1024, T64_DMA), (4096, 4096, 4096, T256_DMA),
                                        (2048, 2048, 4096, T128_DMA), (1536, 1536, 3072, T128_DMA),
                                        (256, 256, 256, T64_DMA), (512, 2048, 1024, T64_DMA),
                                        (2048, 1024, 1024, T128_DMA)])
def test_main_tile_rule(M, N, K, tile):
    # The 64x128 LDS-DMA tile up to a quarter wave of 128x128 tiles, the
    # 128x128 LDS-DMA tile below 80 tiles of 256x256, the 256x256 tile from
    # there on (256 compute units).
    p = plan(M, N, K)
    assert (p.variant, p.tile_id, p.split_k) == (MAIN, tile, 1)


def test_tile_rule_scales_with_the_compute_units():
    # 64 tiles of 256 x 256: under 80 on 256 compute units, past 40 on 128.
    assert plan(2048, 2048, 1024, cus=256).tile_id == T128_DMA
    assert plan(2048, 2048, 1024, cus=128).tile_id == T256_DMA
    # 64 tiles of 128 x 128: a quarter wave on 256 compute units, more on 128.
    assert plan(1024, 1024, 1024, cus=256).tile_id == T64_DMA
    assert plan(1024, 1024, 1024, cus=128).tile_id == T128_DMA


def test_layouts_the_128x128_dma_tile_does_not_take():
    # An N-contiguous B needs N % 8 == 0 on the DMA tiles: the register tile
    # takes it (16-byte rows of 2056 halves holding N = 2052).
    p = plan(1000, 2052, 2048, ldb=2056)
    assert (p.tile_id, p.b_path) == (T128, RVEC)


@pytest.mark.parametrize("M,N,K,variant,split,tile", [
    (1024, 1024, 2048, SPLITK, 4, T128_DMA), (768, 768, 2048, SPLITK, 4, T128_DMA),
    (1024, 1024, 4096, SPLITK, 4, T128_DMA), (512, 512, 2048, SPLITK, 4, T128_DMA),
    (1024, 2048, 2048, SPLITK, 2, T128_DMA), (1024, 1024, 8192, SPLITK, 4, T128_DMA),
    (96, 8192, 8192, SPLITK, 4, T128_DMA), (128, 4096, 8192, SPLITK, 8, T128_DMA),
    (128, 128, 65536, SPLITK, 64, T128_DMA), (256, 256, 16384, SPLITK, 32, T128_DMA),
    (200, 4096, 32768, SPLITK, 8, T128_DMA),      # M < 256, ranges of 8192 k: two per compute unit
    (512, 512, 65536, SPLITK, 40, T256_DMA),      # ranges of 4096 k and more: the 256x256 tile
    (1024, 1024, 16384, SPLITK, 16, T256_DMA), (1024, 2048, 8192, SPLITK, 5, T256_DMA),
    (1024, 1024, 1024, MAIN, 1, T64_DMA), (1024, 1024, 1536, MAIN, 1, T64_DMA),
    (512, 512, 1024, MAIN, 1, T64_DMA), (256, 256, 768, MAIN, 1, T64_DMA),
    (2048, 1024, 1024, MAIN, 1, T128_DMA)])
def test_split_k_rule(M, N, K, variant, split, tile):
    # Operands the 128x128 LDS-DMA tile reads: split-K from K >= 2048 while
    # the 128x128 tiles fill at most half the compute units.  On that tile
    # while its K ranges, one workgroup per compute unit, stay within 2048 k
    # (always with M or N under 256, then two per compute unit once the
    # ranges reach 4096 k); K ranges of at least 512 k.  Longer ranges run
    # on the 256x256 tile, five eighths of a workgroup per compute unit.
    p = plan(M, N, K)
    assert (p.variant, p.split_k, p.tile_id) == (variant, split, tile)
    if variant == SPLITK:
        assert p.workspace_bytes == split * M * N * 4 and p.grid <= 512
        # split counts of 8 or more keep each K range's tiles on one XCD
        assert split < 8 or split % 8 == 0


def test_split_k_rule_for_operands_the_dma_tiles_do_not_read():
    # A with unaligned rows (and N < 256: no realigning copy): split-K from
    # K >= 2 max(M, N), two workgroups per compute unit on the register tile.
    p = plan(512, 200, 2048, lda=2049)
    assert (p.variant, p.tile_id, p.split_k, p.a_path) == (SPLITK, T128, 16, GATHER)
    p = plan(512, 200, 1000, lda=1001)
    assert (p.variant, p.tile_id) == (MAIN, T128)
    # With N >= 256 the same A is realigned, and the split runs on the
    # 128x128 LDS-DMA tile.
    p = plan(1024, 1024, 2048, lda=2049)
    assert (p.variant, p.tile_id, p.split_k, p.a_path) == (SPLITK, T128_DMA, 4, PACKED)


def test_split_k_512x512x65536_grid():
    p = plan(512, 512, 65536)
    assert (p.grid, p.grid2 > 0) == (4 * 40, True)


def test_stream_k_rules():
    p = plan(4352, 4096, 8192)                  # 17 x 16 = 272 tiles: a last wave of 16
    assert (p.variant, p.sk_tiles, p.grid) == (STREAMK, 16, 256)
    p = plan(12288, 2048, 7168)                 # 384 tiles: a last wave of 128, half full
    assert (p.variant, p.sk_tiles) == (STREAMK, 128)
    p = plan(12544, 2048, 7168)                 # 392 tiles: a last wave of 136, over half
    assert (p.variant, p.sk_tiles) == (MAIN, 0)
    p = plan(1536, 1536, 8192)                  # 36 tiles under half a wave, long K: all tiles
    assert (p.variant, p.sk_tiles, p.grid) == (STREAMK, 36, 0)
    p = plan(2048, 2048, 8192)                  # 64 tiles: all in the tail from K = 8192
    assert (p.variant, p.sk_tiles, p.grid) == (STREAMK, 64, 0)
    p = plan(2048, 2048, 6144)                  # below: the 128x128 LDS-DMA tile
    assert (p.variant, p.tile_id) == (MAIN, T128_DMA)
    p = plan(131072, 2048, 7168)                # 16 whole waves
    assert (p.variant, p.tile_id, p.sk_tiles) == (MAIN, T256_DMA, 0)


@pytest.mark.parametrize("M,b,tile_m,b_path", [(1, "row", 16, RVEC), (16, "row", 16, RVEC), (33, "row", 64, RVEC),
                                               (64, "row", 64, RVEC), (16, "nk", 16, KVEC)])
def test_decode_plans(M, b, tile_m, b_path):
    p = plan(M, 2048, 7168, b=b)
    assert (p.variant, p.tile_m, p.tile_n, p.b_path, p.split_k, p.grid) == (SKINNY, tile_m, 128, b_path, 16, 256)


def test_skinny_tiles_take_kcontiguous_b_past_16_rows():
    p = plan(32, 2048, 7168, b="nk")
    assert (p.variant, p.tile_id, p.b_path) == (SKINNY, 4, KVEC)


@pytest.mark.parametrize("M,N,K,a,lda,realigned", [
    (2048, 2048, 2100, "row", None, True),       # rows of 2100 halves
    (2085, 2056, 2051, "strided", None, True),
    (2048, 2048, 2048, "mc", None, True),        # M-contiguous from 2^33 multiply-adds
    (1024, 1024, 1024, "mc", None, False),       # below: the 128 x 128 tile's transposing loads
    (300, 256, 1001, "row", None, False),        # below 2^27: no copy
    (2048, 200, 2100, "row", None, False),       # N under 256
    (2048, 2048, 2048, "row", 2056, False)])     # aligned rows need no copy
def test_realigning_rule(M, N, K, a, lda, realigned):
    p = plan(M, N, K, a=a, lda=lda)
    if realigned:
        assert p.a_path == PACKED and p.workspace_bytes >= M * (-(-K // 64) * 64) * 2, p.as_dict()
    else:
        assert p.a_path != PACKED, p.as_dict()
        assert p.workspace_bytes == (p.split_k * M * N * 4 if p.split_k > 1 else 0), p.as_dict()


@pytest.mark.parametrize("M,N,K,b,ldb,variant,packed", [
    (2048, 2100, 2048, "row", None, MAIN, True),        # rows of 2100 halves, from 1024 rows
    (1000, 4100, 2048, "row", None, MAIN, False),       # under 1024 rows: element-wise on 128 x 128
    (512, 515, 16384, "row", None, SPLITK, True),       # split-K from M, N >= 256
    (16384, 2048, 7168, "nk", None, MAIN, True),        # K-contiguous B from 16384 rows
    (8192, 2048, 7168, "nk", None, MAIN, False)])       # below: the direct K-major stages
def test_packing_rule(M, N, K, b, ldb, variant, packed):
    p = plan(M, N, K, b=b, ldb=ldb)
    assert p.variant == variant, p.as_dict()
    assert (p.b_path == PACKED) == packed, p.as_dict()
    if packed:
        assert p.tile_id == T256_DMA and p.workspace_bytes >= g.lib.gemm_f16_packed_b_bytes(K, N)


def test_unreadable_b_keeps_its_path_without_the_128x128_alternative():
    # Under 1024 rows nothing is packed; the plan reads B element by element.
    p = plan(1000, 4100, 2048)
    assert (p.tile_id, p.b_path) == (T128, GATHER)


def test_forced_options_take_no_copies():
    # Only automatic plans pack or realign.
    o = _lib.Opts(1, 0, 0, 0)
    p = plan(2048, 2100, 2100, opts=o)
    assert (p.a_path, p.b_path, p.workspace_bytes) == (GATHER, GATHER, 0)


# ------------------------------------------------------------------ FP8 (gemm_f8_plan_cus)

def plan8(M, N, K, b="nk", cus=256, opts=None):
    """FP8 A [M, K] K-contiguous (rows padded to 16 bytes); B as [N, K] rows
    ("nk") or [K, N] rows ("kn", N % 16 == 0)."""
    lda = K + (-K) % 16
    ldb_k, ldb_n = (1, lda) if b == "nk" else (N, 1)
    info = _lib.PlanInfo()
    rc = g.lib.gemm_f8_plan_cus(PA, lda, 1, PB, ldb_k, ldb_n, PC, N, M, N, K, 0, 0, cus,
                                ctypes.byref(opts) if opts else None, ctypes.byref(info))
    assert rc == 0, rc
    return info


@pytest.mark.parametrize("M,N,K,b,variant,tile,split", [
    (1, 2048, 7168, "kn", SKINNY, 3, 16), (32, 2048, 7168, "kn", SKINNY, 3, 16),   # decode kernel
    (1, 2048, 7168, "nk", SKINNY, 3, 16), (16, 2048, 7168, "nk", SKINNY, 3, 16),
    (33, 2048, 7168, "kn", SPLITK, 15, 14),      # beyond the decode bound, [K, N] rows: the FP8 tile
    (17, 2048, 7168, "nk", SPLITK, 7, 8),        # [N, K] rows: split on the 128 x 128 LDS-DMA tile
    (1024, 1024, 1024, "nk", MAIN, 8, 1), (1024, 1024, 2048, "nk", MAIN, 8, 1),
    (2048, 2048, 2048, "nk", MAIN, 7, 1), (3072, 3072, 3072, "nk", MAIN, 15, 1),
    (1024, 1024, 8192, "nk", SPLITK, 7, 4), (2048, 2048, 2048, "kn", MAIN, 15, 1),
    (2048, 2048, 2049, "nk", MAIN, 15, 1)])     # odd K: no byte pairs
def test_f8_rules(M, N, K, b, variant, tile, split):
    p = plan8(M, N, K, b)
    assert (p.variant, p.tile_id, p.split_k) == (variant, tile, split), (p.variant, p.tile_id, p.split_k)


def test_f8_compute_unit_count_is_checked():
    info = _lib.PlanInfo()
    for cus in (0, 65537):
        assert g.lib.gemm_f8_plan_cus(PA, 64, 1, PB, 1, 64, PC, 64, 64, 64, 64, 0, 0, cus, None,
                                      ctypes.byref(info)) == -7
    assert g.lib.gemm_f8_plan_cus(PA, 64, 1, PB, 1, 64, PC, 64, 64, 64, 64, 2, 0, 256, None,
                                  ctypes.byref(info)) == -7        # format 2 does not exist
