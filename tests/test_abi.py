"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects every argument outside the contract before touching a
device (so no GPU is needed).  No compute call is made here."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_tiled_gemm_fp16_amd as g
from dense_tiled_gemm_fp16_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16.h")

# Aligned, non-overlapping stand-in device addresses: validation never
# dereferences them.
PA, PB, PC, PW = 0x7F0000000000, 0x7F4000000000, 0x7F8000000000, 0x7FC000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gemm_(?:b?f16|f8)\w*)\s*\(", text,
                                 re.M)))


def test_header_declares_the_binding_list():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(g.lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_status_strings_and_version():
    for rc, name in _lib.STATUS.items():
        s = g.lib.gemm_f16_status_string(rc).decode()
        assert s and s != "unknown status", name
    assert g.lib.gemm_f16_status_string(12345).decode() == "unknown status"
    assert g.lib.gemm_f16_version() >= 100


def call(A=PA, lda_m=64, lda_k=1, B=PB, ldb_k=32, ldb_n=1, C=PC, ldc=32, M=16, N=32, K=64,
         ws=0, ws_bytes=0, opts=None):
    return g.gemm_raw(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, 0, ws, ws_bytes, opts)


@pytest.mark.parametrize("kw,code", [
    (dict(A=0), -1), (dict(B=0), -1), (dict(C=0), -1),
    (dict(M=0), -2), (dict(N=0), -2), (dict(K=0), -2), (dict(M=-3), -2),
    (dict(lda_m=0), -3), (dict(lda_k=-1), -3), (dict(ldb_k=0), -3), (dict(ldb_n=-2), -3),
    (dict(ldc=31), -4),
    (dict(C=PA + 64), -5),                      # C starts inside A
    (dict(C=PB - 64), -5),                      # C runs into B
    (dict(lda_m=2 ** 62, M=4), -2),             # span overflows int64
    (dict(ldb_k=2 ** 61, K=9), -2),
])
def test_rejected_before_any_device_work(kw, code):
    assert call(**kw) == code


def test_option_errors():
    bad = [_lib.Opts(9, 0, 0, 0), _lib.Opts(-1, 0, 0, 0), _lib.Opts(3, -1, 0, 0),
           _lib.Opts(3, 257, 0, 0), _lib.Opts(1, 0, -2, 0), _lib.Opts(1, 0, 5000, 0),
           _lib.Opts(1, 0, 0, 99)]
    for o in bad:
        assert call(opts=o) == -7
    # skinny is only for M <= 64; main takes no K split
    assert call(M=65, opts=_lib.Opts(2, 4, -1, 0)) == -7
    assert call(opts=_lib.Opts(1, 4, 8, 0)) == -7
    # stream-K runs on the 256x256 LDS-DMA tile only, and variants end at 5
    assert call(opts=_lib.Opts(6, 0, 0, 0)) == -7
    assert call(opts=_lib.Opts(5, 0, 0, 1)) == -7
    assert call(lda_m=1, lda_k=64, opts=_lib.Opts(5, 0, 0, 0)) == -7   # A not K-contiguous


def test_forced_tile_without_16_bit_kernels_is_an_option_error():
    # Tile 15 holds FP8 kernels only and ids 9-12 are unused: a call that
    # forces a tile without kernels for its format returns at once with
    # GEMM_ERR_OPTS under every variant.  It runs in a child process with a time limit, so a
    # planning loop fails the test instead of hanging the suite.
    code = (
        "import ctypes, itertools, dense_tiled_gemm_fp16_amd as g\n"
        "from dense_tiled_gemm_fp16_amd import _lib\n"
        "info = _lib.PlanInfo()\n"
        "for v, t in itertools.product((0, 1, 2, 3, 5), (9, 10, 11, 12, 15)):\n"
        "    o = _lib.Opts(v, 0, 0, t)\n"
        "    for f in (g.lib.gemm_f16_plan, g.lib.gemm_bf16_plan):\n"
        f"        print(v, t, f({PA}, 64, 1, {PB}, 32, 1, {PC}, 32, 16, 32, 64, ctypes.byref(o), ctypes.byref(info)))\n"
        f"    print(v, t, g.gemm_raw({PA}, 64, 1, {PB}, 32, 1, {PC}, 32, 16, 32, 64, 0, 0, 0, o))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=ROOT)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.split("\n")[:-1]
    assert len(lines) == 5 * 5 * 3
    for line in lines:
        assert line.split()[2] == "-7", line


def test_workspace_errors():
    o = _lib.Opts(3, 4, -1, 1)                  # forced split-K: no device query needed
    need = g.workspace_bytes(16, 32, 1024, variant="splitk", split_k=4, panel=-1, tile=1)
    assert need == 4 * 16 * 32 * 4
    kw = dict(K=1024, lda_m=1024, opts=o)
    assert call(ws=PW, ws_bytes=need - 1, **kw) == -6
    assert call(ws=PW + 16, ws_bytes=need, **kw) == -6        # not 256-byte aligned
    assert call(ws=PA, ws_bytes=need, **kw) == -5             # overlaps A


def forced_plan(M, N, K, lda, ldb, ldc, variant, split, panel, tile, A=PA, B=PB, C=PC):
    info = _lib.PlanInfo()
    o = _lib.Opts(variant, split, panel, tile)
    rc = g.lib.gemm_f16_plan(A, lda[0], lda[1], B, ldb[0], ldb[1], C, ldc, M, N, K,
                             ctypes.byref(o), ctypes.byref(info))
    assert rc == 0, rc
    return info


def test_plan_of_the_pages_edge_geometry():
    # 130x70x65 with the 64x32x32 tile: a 3x3 grid (Triton article, section
    # "three dimensions that do not divide"); rows of 65 and 70 halves are not
    # 16-byte multiples, so both operands take the element-wise path.
    p = forced_plan(130, 70, 65, (65, 1), (70, 1), 70, 4, 0, -1, 0)
    assert (p.tile_m, p.tile_n, p.tile_k) == (64, 32, 32)
    assert p.grid == 9 and p.split_k == 1 and p.workspace_bytes == 0
    assert (p.a_path, p.b_path) == (0, 0)


def test_plan_paths_follow_strides_and_alignment():
    # A K-contiguous and B N-contiguous (the row-major case)
    p = forced_plan(4096, 4096, 4096, (4096, 1), (4096, 1), 4096, 1, 0, 8, 1)
    assert (p.a_path, p.b_path) == (1, 2) and p.grid == 32 * 32
    # B as a transposed view (stride (1, K)): K-contiguous too
    p = forced_plan(4096, 1061, 8192, (8192, 1), (1, 8192), 1061, 1, 0, 8, 1)
    assert (p.a_path, p.b_path) == (1, 1)
    # A as a transposed view: M-contiguous
    p = forced_plan(256, 256, 256, (1, 256), (256, 1), 256, 1, 0, 8, 1)
    assert (p.a_path, p.b_path) == (2, 2)
    # misaligned base falls back to the element-wise path
    p = forced_plan(256, 256, 256, (256, 1), (256, 1), 256, 1, 0, 8, 1, A=PA + 2)
    assert p.a_path == 0


def test_plan_split_k_extents():
    p = forced_plan(512, 512, 65536, (65536, 1), (512, 1), 512, 3, 16, -1, 1)
    assert p.split_k == 16 and p.grid == 16 * 16 and p.grid2 > 0
    assert p.workspace_bytes == 16 * 512 * 512 * 4
    # the split count never leaves an empty K range
    p = forced_plan(512, 512, 100, (100, 1), (512, 1), 512, 3, 7, -1, 1)
    assert p.split_k == 2          # K = 100 in 64-wide steps: two ranges at most


# ---------------------------------------------------------------- grouped entry point

PO = 0x7E0000000000            # stand-in device address of the offsets


def gcall(A=PA, lda_m=64, lda_k=1, B=PB, ldb_g=64 * 32, ldb_k=32, ldb_n=1, C=PC, ldc=32,
          off=PO, G=4, M=16, N=32, K=64, ws=0, ws_bytes=0):
    return g.lib.gemm_f16_grouped(A, lda_m, lda_k, B, ldb_g, ldb_k, ldb_n, C, ldc, off, G, M, N,
                                  K, 0, ws, ws_bytes)


@pytest.mark.parametrize("kw,code", [
    (dict(off=0), -1), (dict(A=0), -1), (dict(B=0), -1), (dict(C=0), -1),
    (dict(G=0), -2), (dict(G=(1 << 20) + 1), -2), (dict(M=0), -2), (dict(K=-1), -2),
    (dict(ldb_g=-1), -3), (dict(lda_k=0), -3), (dict(ldb_n=0), -3),
    (dict(ldc=31), -4),
    (dict(C=PB + 3 * 64 * 32 * 2 + 64), -5),   # C inside the last group's B
    (dict(C=PA + 2), -5),
    (dict(ldb_g=2 ** 61, G=9), -2),             # B's span overflows int64
])
def test_grouped_rejected_before_any_device_work(kw, code):
    assert gcall(**kw) == code


def test_grouped_workspace():
    need = g.lib.gemm_f16_grouped_workspace_bytes(4)
    assert need == 256                          # 16 * (G + 1) bytes, rounded up to 256
    assert g.lib.gemm_f16_grouped_workspace_bytes(0) == 0
    assert g.lib.gemm_f16_grouped_workspace_bytes(1000) == (16 * 1001 + 255) // 256 * 256
    assert gcall(ws=PW, ws_bytes=need - 1) == -6
    assert gcall(ws=PW + 16, ws_bytes=need) == -6
    assert gcall(ws=PC, ws_bytes=need) == -5    # workspace overlapping C


def test_bf16_options_and_plans():
    def bcall(o):
        return g.lib.gemm_bf16_ex(PA, 64, 1, PB, 32, 1, PC, 32, 16, 32, 64, 0, 0, 0, o)
    assert bcall(_lib.Opts(4, 0, 0, 0)) == -7      # the 64x32x32 variant is fp16-only
    assert bcall(_lib.Opts(1, 0, 4, 11)) == -7     # a tile without bfloat16 kernels
    for tile in (2, 6, 13, 15):                    # fp16-only (2, 6, 13) and FP8-only (15)
        assert bcall(_lib.Opts(1, 0, 4, tile)) == -7, tile
    assert bcall(_lib.Opts(1, 0, 4, 99)) == -7
    info = _lib.PlanInfo()
    for tile in (7, 8, 14, 1):                     # bfloat16 kernels: forced tiles plan on the CPU
        rc = g.lib.gemm_bf16_plan(PA, 1024, 1, PB, 512, 1, PC, 512, 300, 512, 1024,
                                  ctypes.byref(_lib.Opts(1, 0, 4, tile)), ctypes.byref(info))
        assert rc == 0 and info.tile_id == tile, (tile, rc, info.tile_id)
    info = _lib.PlanInfo()
    o = _lib.Opts(3, 4, -1, 1)                     # forced split-K on the 128x128 tile
    rc = g.lib.gemm_bf16_plan(PA, 1024, 1, PB, 32, 1, PC, 32, 16, 32, 1024, ctypes.byref(o),
                              ctypes.byref(info))
    assert rc == 0 and info.split_k == 4 and info.workspace_bytes == 4 * 16 * 32 * 4
    assert g.lib.gemm_bf16_workspace_bytes(16, 32, 1024, ctypes.byref(o)) == 4 * 16 * 32 * 4


def f8call(A=PA, lda_m=64, lda_k=1, B=PB, ldb_k=1, ldb_n=64, C=PC, ldc=32, M=16, N=32, K=64,
           fa=0, fb=0, opts=None):
    return g.lib.gemm_f8_ex(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, fa, fb, 0, 0, 0,
                            ctypes.byref(opts) if opts is not None else None)


def test_f8_rejected_before_any_device_work():
    # Layout: K-contiguous A and B with 16-byte aligned rows only.
    assert f8call(lda_m=1, lda_k=64) == -9              # A not K-contiguous
    assert f8call(ldb_k=32, ldb_n=1) != -9              # B N-contiguous, N % 16 == 0: taken
    assert f8call(ldb_k=40, ldb_n=1) == -9              # its k-rows not 16-byte aligned
    assert f8call(ldb_k=32, ldb_n=1, N=24, ldc=24) == -9   # N not a multiple of 16
    assert f8call(ldb_k=32, ldb_n=2) == -9              # B contiguous along neither axis
    assert f8call(ldb_k=(1 << 24) + 16, ldb_n=1) == -9  # k-rows over 2^24 bytes apart
    assert f8call(lda_m=72) == -9                       # A rows not 16-byte aligned
    assert f8call(ldb_n=40) == -9
    assert f8call(A=PA + 8) == -9
    assert f8call(lda_m=(1 << 24) + 16) == -9           # rows over 2^24 bytes apart
    assert f8call(ldb_n=(1 << 24) + 16) == -9
    assert f8call(fa=2) == -7 and f8call(fb=-1) == -7   # formats 0 (E4M3) and 1 (E5M2)
    # skinny FP8 (the decode kernel): up to 16 rows with B as [N, K] rows, 64
    # with [K, N] rows, no forced tile
    assert f8call(M=17, opts=_lib.Opts(2, 0, 0, 0)) == -7
    assert f8call(M=65, ldb_k=32, ldb_n=1, opts=_lib.Opts(2, 0, 0, 0)) == -7
    assert f8call(opts=_lib.Opts(2, 0, 0, 15)) == -7
    assert f8call(opts=_lib.Opts(4, 0, 0, 0)) == -7
    assert f8call(opts=_lib.Opts(1, 0, 0, 14)) == -7    # the FP8 tile only
    assert f8call(M=0) == -2 and f8call(ldc=31) == -4 and f8call(A=0) == -1
    # byte-sized A and B: C may start right after A's last byte
    assert f8call(C=PA + 15 * 64 + 64) != -5
    assert f8call(C=PA + 15 * 64 + 62) == -5


def test_f8_plans():
    info = _lib.PlanInfo()
    for fa, fb in ((0, 0), (0, 1), (1, 0), (1, 1)):
        rc = g.lib.gemm_f8_plan(PA, 704, 1, PB, 1, 704, PC, 520, 600, 520, 700, fa, fb,
                                ctypes.byref(_lib.Opts(1, 0, 4, 15)), ctypes.byref(info))
        assert rc == 0
        assert (info.tile_id, info.tile_m, info.tile_n, info.tile_k) == (15, 256, 256, 64)
        assert (info.split_k, info.grid, info.workspace_bytes) == (1, 9, 0)
    for tile in (15, 7, 8):                 # forced tiles plan without the device
        rc = g.lib.gemm_f8_plan(PA, 704, 1, PB, 1, 704, PC, 520, 600, 520, 700, 0, 0,
                                ctypes.byref(_lib.Opts(3, 3, -1, tile)), ctypes.byref(info))
        assert rc == 0 and info.split_k == 3 and info.workspace_bytes == 3 * 600 * 520 * 4
        assert info.tile_id == tile
        assert g.lib.gemm_f8_workspace_bytes(600, 520, 700, ctypes.byref(_lib.Opts(3, 3, -1, tile))) \
            == info.workspace_bytes
    # the 128-wide tiles read FP8 byte pairs of K-contiguous B: B [K, N] rows
    # or an odd K hand over to the FP8 tile
    rc = g.lib.gemm_f8_plan(PA, 704, 1, PB, 528, 1, PC, 528, 600, 528, 700, 0, 0,
                            ctypes.byref(_lib.Opts(1, 0, 4, 7)), ctypes.byref(info))
    assert rc == 0 and info.tile_id == 15
    rc = g.lib.gemm_f8_plan(PA, 704, 1, PB, 1, 704, PC, 520, 600, 520, 701, 0, 0,
                            ctypes.byref(_lib.Opts(1, 0, 4, 8)), ctypes.byref(info))
    assert rc == 0 and info.tile_id == 15


def test_packed_b_rejected_before_any_device_work():
    nb = g.lib.gemm_f16_packed_b_bytes(100, 300)
    assert nb == 2 * 4 * 16384                                      # 2 panels x 4 blocks of 32 k
    assert g.lib.gemm_f16_packed_b_bytes(0, 5) == 0
    pack = g.lib.gemm_f16_pack_b
    assert pack(0, 300, 1, 100, 300, PW, 0) == -1
    assert pack(PB, 300, 1, 0, 300, PW, 0) == -2
    assert pack(PB, 0, 1, 100, 300, PW, 0) == -3
    assert pack(PB, 300, 1, 100, 300, PW + 16, 0) == -6             # Bp not 256-byte aligned
    assert pack(PB, 300, 1, 100, 300, PB + 256, 0) == -5            # Bp overlaps B
    run = g.lib.gemm_f16_packed
    assert run(PA, 100, 1, PW, PC, 300, 50, 300, 100, 0) == -9      # A rows not 16-byte multiples
    assert run(PA, 1, 50, PW, PC, 300, 50, 300, 100, 0) == -9       # A not K-contiguous
    assert run(PA, (1 << 23) + 8, 1, PW, PC, 300, 50, 300, 100, 0) == -9   # rows over 2^23 apart
    assert run(PA, 112, 1, PW, PC, 299, 50, 300, 100, 0) == -4
    assert run(PA, 112, 1, PW, PW + 1024, 300, 50, 300, 100, 0) == -5   # C overlaps Bp


def f8gcall(A=PA, lda_m=64, lda_k=1, B=PB, ldb_g=32 * 64, ldb_k=1, ldb_n=64, C=PC, ldc=32,
            off=PO, G=4, M=16, N=32, K=64, fa=0, fb=1, ws=PW, ws_bytes=255):
    """gemm_f8_grouped with byte strides; by default B_g K-contiguous ([N, K]
    rows of 64 bytes) and a workspace one byte short, so a call whose
    layout is accepted stops at the workspace check (-6), before any launch."""
    return g.lib.gemm_f8_grouped(A, lda_m, lda_k, B, ldb_g, ldb_k, ldb_n, C, ldc, off, G, M, N, K,
                                 fa, fb, 0, ws, ws_bytes)


@pytest.mark.parametrize("kw,code", [
    (dict(), -6),                                    # layout accepted
    (dict(ldb_k=64, ldb_n=1, N=32), -6),             # N-contiguous B, N a multiple of 16
    (dict(fa=2), -7), (dict(fb=-1), -7),             # not an FP8 format
    (dict(lda_k=2, lda_m=128), -9),                  # A not K-contiguous
    (dict(lda_m=72), -9),                            # A rows not 16-byte multiples
    (dict(A=PA + 8), -9), (dict(B=PB + 8), -9),      # unaligned bases
    (dict(ldb_g=32 * 64 + 8), -9),                   # a group's B off the 16-byte grid
    (dict(ldb_k=48, ldb_n=1, N=40, ldc=40), -9),     # N-contiguous B, N % 16 != 0
    (dict(ldb_k=2, ldb_n=64), -9),                   # B contiguous along neither axis
    (dict(lda_m=(1 << 24) + 16, M=2), -9),           # row stride past 2^24 bytes
])
def test_f8_grouped_layouts_checked_before_any_device_work(kw, code):
    assert f8gcall(**kw) == code
