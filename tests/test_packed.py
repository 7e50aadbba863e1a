"""GPU parity of the pre-packed static B path (gemm_f16_pack_b +
gemm_f16_packed; the C500 log's weight packing done once, outside the timed
region) against the oracle, and against the general-stride path on integer
inputs.  B is packed from several layouts; padding of A rows is NaN.
"""
import ctypes

import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, ORACLE_THREADS, Out, assert_bits_equal, assert_close, band_rows, dev_nan,
                      place, say,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


def reference(A, B, rows=None):
    K, N = B.shape
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (N, 1), A.shape[0], N, K, nthreads=ORACLE_THREADS)


def run(a, packed, out):
    say(f"gemm_packed M={a.shape[0]} N={packed.N} K={packed.K} a.stride={a.stride()}")
    g.gemm_packed(a, packed, out=out.view)
    torch.cuda.synchronize()
    return out.result()


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("b_layout", ["row", "col", "strided"])
@pytest.mark.parametrize("shape", [(300, 264, 100), (600, 520, 700), (257, 300, 31), (64, 8, 2048)])
def test_packed_parity(shape, b_layout, mode):
    M, N, K = shape
    A = synth.matrix(M, K, 15000 + K, 0, mode)
    B = synth.matrix(K, N, 15000 + N, 1, mode)
    ref = reference(A, B)
    if b_layout == "strided":      # every other column of a wider row-major buffer
        wide = np.zeros((K, 2 * N), dtype=np.uint16)
        wide[:, ::2] = B
        b = to_dev(wide)[:, ::2]
    else:
        b = place(B, b_layout, (1, 3))
    say(f"pack_b K={K} N={N} b.stride={b.stride()}")
    packed = g.pack_b(b)
    a = place(A, "row", (1, (-K) % 8 + 8))
    got = run(a, packed, Out(M, N))
    what = f"packed {shape} B={b_layout} {mode}"
    if mode == "int":
        assert_bits_equal(got, ref, what)
        general = to_host(g.gemm(a, b))
        assert_bits_equal(got, general, what + " vs general path")
    else:
        assert_close(got, ref, what)


def test_packed_moe_shape_sampled():
    M, N, K = 131072, 2048, 7168
    say("packed MoE: generating inputs")
    A = synth.matrix(M, K, 15100, 0)
    B = synth.matrix(K, N, 15101, 1)
    a, b = to_dev(A), to_dev(B)
    packed = g.pack_b(b)
    del b
    c = g.gemm_packed(a, packed)
    torch.cuda.synchronize()
    got = to_host(c)
    rng = np.random.default_rng(15100)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    assert_close(got[rows], reference(A, B, rows), "packed MoE sampled rows")


# ---- automatic packing plan: K-contiguous B at large M (gemm_f16_ex, AUTO)

def _kcontig_case(M, N, K, seed, fmt="f16"):
    A = synth.matrix(M, K, seed, 0, "int", fmt=fmt)
    B = synth.matrix(K, N, seed, 1, "int", fmt=fmt)
    a = place(A, "row", (1, (-K) % 8 + 8))
    b = place(B, "col", (1, (-K) % 8 + 8))     # transposed view: K-contiguous, aligned rows
    if fmt == "bf16":
        a, b = a.view(torch.bfloat16), b.view(torch.bfloat16)
    return A, B, a, b


def _out(M, N, fmt):
    out = Out(M, N)
    if fmt == "bf16":
        out.view = out.view.view(torch.bfloat16)
    return out


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_auto_packs_kcontig_b(fmt):
    # M past the packing threshold with ragged M, N and K (K tail 700 % 64 = 60).
    M, N, K = 16384 + 37, 300, 700
    A, B, a, b = _kcontig_case(M, N, K, 15200, fmt)
    p = g.plan(a, b)
    assert p["b_path"] == "packed" and p["tile_id"] == 14 and p["split_k"] == 1, p
    assert p["workspace_bytes"] == g.lib.gemm_f16_packed_b_bytes(K, N), p
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS,
                      dtype="bf16" if fmt == "bf16" else "f16")
    say(f"auto packing plan {fmt} {M}x{N}x{K} B stride {b.stride()}")
    out = _out(M, N, fmt)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    assert_bits_equal(out.result(), ref, f"packing plan {fmt}")
    say(f"forced direct plan {fmt} {M}x{N}x{K}")
    pd = g.plan(a, b, variant="main", tile=14)
    assert pd["b_path"] == "kvec" and pd["workspace_bytes"] == 0, pd
    out2 = _out(M, N, fmt)
    g.gemm(a, b, out=out2.view, variant="main", tile=14)
    torch.cuda.synchronize()
    assert_bits_equal(out2.result(), ref, f"direct K-major plan {fmt}")


def test_auto_pack_caller_workspace():
    M, N, K = 16384, 264, 512
    A, B, a, b = _kcontig_case(M, N, K, 15300)
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS)
    need = int(g.lib.gemm_f16_packed_b_bytes(K, N))
    assert g.plan(a, b)["b_path"] == "packed"
    # Big enough: the packing plan runs in the caller's workspace.
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device=DEV)
    say(f"packing plan in a caller workspace of {need} bytes")
    out = Out(M, N)
    g.gemm(a, b, out=out.view, workspace=ws)
    torch.cuda.synchronize()
    assert_bits_equal(out.result(), ref, "caller workspace")
    assert not torch.isnan(ws[: need // 4]).all()      # the packed B went there
    # Too small: the direct plan runs, same bits, the workspace untouched.
    small = torch.full((1024,), float("nan"), dtype=torch.float32, device=DEV)
    say("packing plan with a too-small caller workspace -> direct plan")
    out2 = Out(M, N)
    g.gemm(a, b, out=out2.view, workspace=small)
    torch.cuda.synchronize()
    assert_bits_equal(out2.result(), ref, "small workspace")
    assert torch.isnan(small).all()


def test_auto_pack_workspace_overlapping_b_rejected():
    M, N, K = 16384, 264, 512
    _, _, a, b = _kcontig_case(M, N, K, 15400)
    need = int(g.lib.gemm_f16_packed_b_bytes(K, N))
    assert g.plan(a, b)["b_path"] == "packed"
    # A workspace that starts inside B's storage: rejected before any launch.
    base = b.data_ptr() - (b.data_ptr() % 256) + 256
    c = torch.empty((M, N), dtype=torch.float16, device=DEV)
    opts = g.make_opts("auto", 0, 0, 0)
    rc = g.lib.gemm_f16_ex(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
                           b.stride(1), c.data_ptr(), N, M, N, K, 0, base, need,
                           ctypes.byref(opts))
    assert rc == -5, rc


def test_auto_pack_moe_shape_sampled():
    M, N, K = 131072, 2048, 7168
    say("K-contiguous B MoE: generating inputs")
    A = synth.matrix(M, K, 15500, 0)
    B = synth.matrix(K, N, 15501, 1)
    a = to_dev(A)
    b = to_dev(np.ascontiguousarray(B.T)).t()        # B as [N, K] weights
    p = g.plan(a, b)
    assert p["b_path"] == "packed", p
    say(f"K-contiguous B MoE plan {p}")
    c = g.gemm(a, b)
    torch.cuda.synchronize()
    got = to_host(c)
    rng = np.random.default_rng(15500)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    assert_close(got[rows], reference(A, B, rows), "K-contiguous B MoE sampled rows")


def test_auto_pack_streamk():
    # 65 x 5 = 325 tiles on 256 compute units: a final wave of 69 tiles, so
    # the automatic plan is stream-K, here with the packed B in front of the
    # partials.  Same split forced without packing must give the same bits.
    M, N, K = 16384 + 37, 1061, 2100
    A, B, a, b = _kcontig_case(M, N, K, 15600)
    p = g.plan(a, b)
    if p["variant"] != "streamk":
        pytest.skip(f"this device's compute-unit count gives no stream-K tail here: {p}")
    assert p["b_path"] == "packed", p
    assert p["workspace_bytes"] > g.lib.gemm_f16_packed_b_bytes(K, N), p
    say(f"stream-K packing plan {p}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    pd = g.plan(a, b, variant="streamk", split_k=p["split_k"])
    assert pd["b_path"] == "kvec" and pd["sk_tiles"] == p["sk_tiles"], pd
    say(f"stream-K direct plan {pd}")
    out2 = Out(M, N)
    g.gemm(a, b, out=out2.view, variant="streamk", split_k=p["split_k"])
    torch.cuda.synchronize()
    assert_bits_equal(got, out2.result(), "stream-K packed vs direct")
    rng = np.random.default_rng(15600)
    rows = np.unique(np.concatenate([[0, 255, 16383, 16384, M - 1], rng.integers(0, M, 8)]))
    assert_bits_equal(got[rows], reference(A, B, rows), "stream-K packing plan sampled rows")


def _gather_b_case(M, N, K, seed, layout):
    A = synth.matrix(M, K, seed, 0, "int")
    B = synth.matrix(K, N, seed, 1, "int")
    a = place(A, "row", (1, (-K) % 8 + 8))
    if layout == "row_unaligned":            # rows of N halves, N odd: not 16-byte aligned
        b = to_dev(B)
    else:                                    # every other column of a wider buffer
        wide = np.zeros((K, 2 * N), dtype=np.uint16)
        wide[:, ::2] = B
        b = to_dev(wide)[:, ::2]
    return A, B, a, b


@pytest.mark.parametrize("layout", ["row_unaligned", "strided"])
def test_auto_packs_b_the_dma_tile_cannot_read(layout):
    # Enough 256 x 256 tiles for half a wave, so the plan takes that tile.
    M, N, K = (8192 + 37, 1061, 700) if layout == "row_unaligned" else (16384 + 37, 300, 700)
    A, B, a, b = _gather_b_case(M, N, K, 15700, layout)
    assert g.plan(a, b, variant="main")["b_path"] == "gather"
    p = g.plan(a, b)
    assert p["b_path"] == "packed" and p["tile_id"] == 14, p
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS)
    say(f"packing plan for a {layout} B {M}x{N}x{K} stride {b.stride()}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    assert_bits_equal(out.result(), ref, f"packing plan, {layout} B")
    # No room in the caller's workspace: the element-wise plan, same bits.
    small = torch.empty(1024, dtype=torch.float32, device=DEV)
    say(f"{layout} B with a too-small workspace")
    out2 = Out(M, N)
    g.gemm(a, b, out=out2.view, workspace=small)
    torch.cuda.synchronize()
    assert_bits_equal(out2.result(), ref, f"element-wise plan, {layout} B")


# ---- automatic realigning plan: an A the DMA tile cannot read (gemm_f16_ex, AUTO)

def _a_view(A, layout):
    """A [M, K] on the GPU inside NaN storage, laid out so that the LDS-DMA
    tile cannot read it: rows of a length that is not a 16-byte multiple,
    every other column of a wider buffer, or M-contiguous."""
    M, K = A.shape
    if layout == "odd_ld":
        return place(A, "row", (1, (3 - K) % 8 + 8))          # row stride = 3 (mod 8)
    if layout == "strided":
        buf = dev_nan((M + 1) * 2 * K)
        v = buf[2 * K:].view(M, 2 * K)[:, ::2]
        v.copy_(to_dev(A))
        return v
    if layout == "mcontig":
        return place(A, "col", (1, 8))
    raise ValueError(layout)


def _without_realign(a, b, M, N, K):
    """The automatic plan again with a caller workspace too small for the
    realigned A (the size the split plans need on aligned operands), which
    must give the plan on A's own layout."""
    small = torch.full((max(256, g.workspace_bytes(M, N, K)) // 4 + 64,), float("nan"),
                       dtype=torch.float32, device=DEV)
    out = Out(M, N)
    g.gemm(a, b, out=out.view, workspace=small)
    torch.cuda.synchronize()
    return out.result()


@pytest.mark.parametrize("layout,shape", [("odd_ld", (2085, 2056, 2051)), ("strided", (2085, 2056, 2051)),
                                          ("mcontig", (2048, 2048, 2048))])
def test_auto_realigns_a_the_dma_tile_cannot_read(layout, shape):
    # Integer inputs keep every fp32 sum exact, so the realigned plan, the
    # plan on A's own layout and the oracle must agree bit for bit.
    M, N, K = shape
    seed = 16000 + len(layout)
    A = synth.matrix(M, K, seed, 0, "int")
    B = synth.matrix(K, N, seed, 1, "int")
    a, b = _a_view(A, layout), to_dev(B)
    p = g.plan(a, b)
    assert p["a_path"] == "packed" and p["b_path"] == "rvec", p
    ldp = -(-K // 64) * 64
    assert p["workspace_bytes"] >= M * ldp * 2, p
    say(f"realigning plan, A {layout} {M}x{N}x{K} stride {a.stride()}: {p}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    rows = band_rows(M)
    assert_bits_equal(got[rows], reference(A, B, rows), f"realigned A {layout}, sampled rows")
    say(f"A {layout}: plan without the realigned A")
    assert_bits_equal(got, _without_realign(a, b, M, N, K), f"realigned A {layout} vs A's own layout")


def test_auto_realigns_a_and_packs_b():
    # Neither operand readable by the DMA (rows of 2100 halves): A realigned,
    # B packed, both in the library's workspace.
    M, N, K = 2100, 2100, 2100
    A = synth.matrix(M, K, 16100, 0, "int")
    B = synth.matrix(K, N, 16101, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    assert (p["a_path"], p["b_path"], p["tile_id"]) == ("packed", "packed", 14), p
    say(f"realigned A and packed B {M}x{N}x{K}: {p}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    rows = band_rows(M)
    assert_bits_equal(got[rows], reference(A, B, rows), "realigned A, packed B, sampled rows")
    assert_bits_equal(got, _without_realign(a, b, M, N, K), "realigned A, packed B vs element-wise")


@pytest.mark.parametrize("shape,variant", [((512, 512, 65539), "splitk"), ((1536, 1536, 8195), "streamk")])
def test_auto_realign_split_plans(shape, variant):
    # Odd K: A's rows are never 16-byte aligned.  The split plans put their
    # partials after the realigned A; integer sums stay exact in fp32
    # (|sum| < 2^24), so any K split gives the oracle's bits.
    M, N, K = shape
    A = synth.matrix(M, K, 16200 + M, 0, "int")
    B = synth.matrix(K, N, 16200 + M, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    if p["variant"] != variant:
        pytest.skip(f"this device's compute-unit count gives another plan here: {p}")
    assert p["a_path"] == "packed", p
    say(f"realigning {variant} plan {M}x{N}x{K}: {p}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    rows = band_rows(M, 128)
    assert_bits_equal(got[rows], reference(A, B, rows), f"realigned A {variant}, sampled rows")
    assert_bits_equal(got, _without_realign(a, b, M, N, K), f"realigned A {variant} vs A's own layout")


def test_auto_realigns_a_bf16():
    # The realigning pass moves 16-bit words, so bfloat16 takes it too.
    M, N, K = 2085, 2056, 2051
    A = synth.matrix(M, K, 16300, 0, "int", fmt="bf16")
    B = synth.matrix(K, N, 16301, 1, "int", fmt="bf16")
    a = _a_view(A, "odd_ld").view(torch.bfloat16)
    b = to_dev(B).view(torch.bfloat16)
    p = g.plan(a, b)
    assert p["a_path"] == "packed", p
    say(f"bf16 realigning plan {M}x{N}x{K}: {p}")
    out = _out(M, N, "bf16")
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    rows = band_rows(M)
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), (K, 1), B, (N, 1), len(rows), N, K,
                      nthreads=ORACLE_THREADS, dtype="bf16")
    assert_bits_equal(got[rows], ref, "bf16 realigned A, sampled rows")
    out2 = _out(M, N, "bf16")
    g.gemm(a, b, out=out2.view, variant="main", tile=1)
    torch.cuda.synchronize()
    assert_bits_equal(got, out2.result(), "bf16 realigned A vs the 128x128 tile on A's own layout")


@pytest.mark.parametrize("layout", ["row_unaligned", "strided"])
def test_auto_split_k_packs_b_the_dma_tile_cannot_read(layout):
    # K >> M, N: the split-K plan packs B for the 256 x 256 tile (its fp32
    # partials after the packed B) rather than read it element by element.
    # Integer sums stay exact in fp32 (|sum| < 2^24), so the packed plan, the
    # element-wise plan and the oracle agree bit for bit.
    M, N, K = (512, 515, 16384) if layout == "row_unaligned" else (520, 300, 12000)
    A, B, a, b = _gather_b_case(M, N, K, 16400, layout)
    p = g.plan(a, b)
    assert (p["variant"], p["b_path"], p["tile_id"]) == ("splitk", "packed", 14), p
    say(f"split-K packing plan, {layout} B {M}x{N}x{K}: {p}")
    out = Out(M, N)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    rows = band_rows(M, 128)
    assert_bits_equal(got[rows], reference(A, B, rows), f"split-K packing plan, {layout} B, sampled rows")
    small = torch.full((max(256, g.workspace_bytes(M, N, K)) // 4 + 64,), float("nan"),
                       dtype=torch.float32, device=DEV)
    out2 = Out(M, N)
    g.gemm(a, b, out=out2.view, workspace=small)
    torch.cuda.synchronize()
    assert_bits_equal(got, out2.result(), f"split-K packing plan vs element-wise plan, {layout} B")
