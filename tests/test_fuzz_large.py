"""Seeded randomized parity at large M, where the automatic plans pack B
(K-contiguous B from M = 16384, a B the LDS-DMA tile cannot read from
M = 1024) and take the stream-K tail; each B layout is drawn three times.
A second set draws mid-size products (M from 1024) with every A and B
layout, where the automatic plans also realign A and split K.  Integer
inputs in [-4, 4] keep every fp32 sum exact.  The automatic plan's output
must have every element written, and agree bit for bit with the oracle on
one row per 256-row band and on 20000 points drawn over the whole output,
and with the forced main plan (never packed) everywhere; the mid-size sets
compare with the 128 x 128 register-path tile, another kernel, instead.  A
third set draws small and mid-size outputs with long K, where the plans
split K on the LDS-DMA tiles.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import DEV, NAN16, ORACLE_THREADS, Out, assert_bits_equal, band_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _b_view(B, layout, fmt):
    K, N = B.shape
    if layout == "row":
        v = to_dev(B)
    elif layout == "col":                      # [N, K] rows, K padded to 8
        ld = K + (-K) % 8
        buf = np.zeros((N, ld), dtype=np.uint16)
        buf[:, :K] = B.T
        v = to_dev(buf)[:, :K].t()
    elif layout == "unaligned":                # rows of N + 1 halves (odd pitch when N is even)
        ld = N + 1 if N % 2 == 0 else N + 2
        buf = np.zeros((K, ld), dtype=np.uint16)
        buf[:, :N] = B
        v = to_dev(buf)[:, :N]
    else:                                      # every other column of a wider buffer
        wide = np.zeros((K, 2 * N), dtype=np.uint16)
        wide[:, ::2] = B
        v = to_dev(wide)[:, ::2]
    return v.view(torch.bfloat16) if fmt == "bf16" else v


def _case(seed):
    rng = np.random.default_rng(seed)
    layout = ["row", "col", "unaligned", "strided"][seed % 4]
    M = int(rng.integers(16384 if layout == "col" else 4096, 32769))   # col: past the packing threshold
    N = int(rng.integers(1, 2201))
    K = int(rng.integers(1, 3001))
    fmt = "bf16" if rng.random() < 0.3 else "f16"
    return M, N, K, layout, fmt


@pytest.mark.parametrize("seed", range(19000, 19012))
def test_random_large_case(seed):
    M, N, K, layout, fmt = _case(seed)
    A = synth.matrix(M, K, seed, 0, "int", fmt=fmt)
    B = synth.matrix(K, N, seed, 1, "int", fmt=fmt)
    ld = K + (-K) % 8
    abuf = np.zeros((M, ld), dtype=np.uint16)
    abuf[:, :K] = A
    a = to_dev(abuf)[:, :K]
    if fmt == "bf16":
        a = a.view(torch.bfloat16)
    b = _b_view(B, layout, fmt)
    p = g.plan(a, b)
    say(f"large fuzz seed={seed} {fmt} {M}x{N}x{K} B={layout} stride={b.stride()} -> {p}")
    out = Out(M, N)
    if fmt == "bf16":
        out.view = out.view.view(torch.bfloat16)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    assert np.all(got != NAN16), f"seed {seed}: outputs never written"
    out2 = Out(M, N)
    if fmt == "bf16":
        out2.view = out2.view.view(torch.bfloat16)
    g.gemm(a, b, out=out2.view, variant="main")
    torch.cuda.synchronize()
    assert_bits_equal(got, out2.result(), f"seed {seed}: automatic plan {p} vs forced main")
    dt = "bf16" if fmt == "bf16" else "f16"
    rows = band_rows(M)
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), (K, 1), B, (N, 1), len(rows), N, K,
                      nthreads=ORACLE_THREADS, dtype=dt)
    assert_bits_equal(got[rows], ref, f"seed {seed}: band rows against the oracle")
    rng = np.random.default_rng(seed + 1)
    pr, pc = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    ref = oracle.gemm_points(A, (K, 1), B, (N, 1), K, pr, pc, nthreads=ORACLE_THREADS, dtype=dt)
    assert_bits_equal(got[pr, pc], ref, f"seed {seed}: points against the oracle")


def _a_view(A, layout, fmt):
    M, K = A.shape
    if layout == "row":                        # K-contiguous rows padded to 8 halves
        ld = K + (-K) % 8
        buf = np.zeros((M, ld), dtype=np.uint16)
        buf[:, :K] = A
        v = to_dev(buf)[:, :K]
    elif layout == "odd":                      # rows of an odd number of halves
        ld = K + 1 if K % 2 == 0 else K + 2
        buf = np.zeros((M, ld), dtype=np.uint16)
        buf[:, :K] = A
        v = to_dev(buf)[:, :K]
    elif layout == "mcontig":                  # A as a transposed view
        ld = M + (-M) % 8
        buf = np.zeros((K, ld), dtype=np.uint16)
        buf[:, :M] = A.T
        v = to_dev(buf)[:, :M].t()
    else:                                      # every other column of a wider buffer
        wide = np.zeros((M, 2 * K), dtype=np.uint16)
        wide[:, ::2] = A
        v = to_dev(wide)[:, ::2]
    return v.view(torch.bfloat16) if fmt == "bf16" else v


@pytest.mark.parametrize("seed", range(19100, 19116))
def test_random_mid_case(seed):
    # Integer inputs keep every sum exact, so the automatic plan (realigned
    # A, packed B, split K or stream-K as the shape and layouts decide) must
    # equal the main plan of the 128 x 128 register-path tile, another
    # kernel, on the operands' own layouts everywhere.
    rng = np.random.default_rng(seed)
    a_layout = ["row", "odd", "mcontig", "strided"][seed % 4]
    b_layout = ["row", "col", "unaligned", "strided"][(seed // 4) % 4]
    M = int(rng.integers(1024, 6145))
    N = int(rng.integers(256, 2305))
    K = int(rng.integers(64, 4097))
    fmt = "bf16" if rng.random() < 0.25 else "f16"
    A = synth.matrix(M, K, seed, 0, "int", fmt=fmt)
    B = synth.matrix(K, N, seed, 1, "int", fmt=fmt)
    a, b = _a_view(A, a_layout, fmt), _b_view(B, b_layout, fmt)
    p = g.plan(a, b)
    say(f"mid fuzz seed={seed} {fmt} {M}x{N}x{K} A={a_layout} B={b_layout} -> {p}")
    out = Out(M, N)
    if fmt == "bf16":
        out.view = out.view.view(torch.bfloat16)
    g.gemm(a, b, out=out.view)
    torch.cuda.synchronize()
    got = out.result()
    assert np.all(got != NAN16), f"seed {seed}: outputs never written"
    out2 = Out(M, N)
    if fmt == "bf16":
        out2.view = out2.view.view(torch.bfloat16)
    g.gemm(a, b, out=out2.view, variant="main", tile=1)
    torch.cuda.synchronize()
    assert_bits_equal(got, out2.result(), f"seed {seed}: automatic plan {p} vs the register tile")
    dt = "bf16" if fmt == "bf16" else "f16"
    rows = band_rows(M)
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), (K, 1), B, (N, 1), len(rows), N, K,
                      nthreads=ORACLE_THREADS, dtype=dt)
    assert_bits_equal(got[rows], ref, f"seed {seed}: band rows against the oracle")


@pytest.mark.parametrize("seed", range(19200, 19216))
def test_random_small_long_k_case(seed):
    # Small and mid-size outputs with long K: the 64 x 128 and 128 x 128
    # LDS-DMA tiles, split-K on them or on the 256 x 256 tile, and stream-K
    # over every tile, as the planner decides.  Integer inputs keep every sum
    # exact: the automatic plan must equal the register tile's main plan
    # everywhere, and sampled rows the oracle.
    rng = np.random.default_rng(seed)
    a_layout = ["row", "row", "odd", "strided"][seed % 4]
    b_layout = ["row", "col", "row", "unaligned"][(seed // 4) % 4]
    M = int(rng.integers(65, 1281))
    N = int(rng.integers(64, 1281))
    if b_layout == "row" and rng.random() < 0.7:
        N = N // 8 * 8 or 8                    # whole 16-byte B rows: the DMA tiles take it
    K = int(rng.integers(1024, 10001))
    fmt = "bf16" if rng.random() < 0.25 else "f16"
    A = synth.matrix(M, K, seed, 0, "int", fmt=fmt)
    B = synth.matrix(K, N, seed, 1, "int", fmt=fmt)
    a, b = _a_view(A, a_layout, fmt), _b_view(B, b_layout, fmt)
    p = g.plan(a, b)
    say(f"small long-K fuzz seed={seed} {fmt} {M}x{N}x{K} A={a_layout} B={b_layout} -> {p}")
    outs = []
    for kw in ({}, dict(variant="main", tile=1)):
        out = Out(M, N)
        if fmt == "bf16":
            out.view = out.view.view(torch.bfloat16)
        g.gemm(a, b, out=out.view, **kw)
        torch.cuda.synchronize()
        outs.append(out.result())
    assert np.all(outs[0] != NAN16), f"seed {seed}: outputs never written"
    assert_bits_equal(outs[0], outs[1], f"seed {seed}: automatic plan {p} vs the register tile")
    dt = "bf16" if fmt == "bf16" else "f16"
    rows = band_rows(M)
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), (K, 1), B, (N, 1), len(rows), N, K,
                      nthreads=ORACLE_THREADS, dtype=dt)
    assert_bits_equal(outs[0][rows], ref, f"seed {seed}: band rows against the oracle")
