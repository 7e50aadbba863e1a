"""GPU parity of the grouped entry point (gemm_f16_grouped) against the
oracle's grouped definition, on the same seeded inputs.

Group g owns rows offsets[g] .. offsets[g+1]-1 of A and C and its own B_g
(synthetic expert weights: tensor id 16 + g).  Outputs are pre-filled with
NaN inside canary bands: rows outside every group must stay NaN, and
nothing outside the view may change.  Acceptance as in test_parity:
bit-exact on integer inputs, the elementwise tolerance on U(-1, 1).
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, NAN16, ORACLE_THREADS, Out, assert_bits_equal, assert_close,
                      assert_close_bf16, place,
                      say, to_dev, to_host)

pytestmark = pytest.mark.gpu


def experts(G, K, N, seed, mode, layout):
    """Host [G, K, N] stack and its device view: "row" stores each B_g
    row-major; "col" stores each B_g as a transposed view (K-contiguous)."""
    Bs = np.stack([synth.matrix(K, N, seed, 16 + e, mode) for e in range(G)])
    if layout == "row":
        return Bs, to_dev(Bs)
    return Bs, to_dev(np.ascontiguousarray(Bs.transpose(0, 2, 1))).transpose(1, 2)


def run_grouped(a, b, offsets, out, **kw):
    say(f"grouped M={a.shape[0]} K={a.shape[1]} G={b.shape[0]} N={b.shape[2]} "
        f"a.stride={a.stride()} b.stride={b.stride()} offsets={offsets[:4].tolist()}...")
    g.gemm_grouped(a, b, offsets, out=out.view, **kw)
    torch.cuda.synchronize()
    return out.result()


def check_groups(got, ref, offsets, mode, what):
    M = got.shape[0]
    inside = np.zeros(M, dtype=bool)
    for e in range(len(offsets) - 1):
        inside[offsets[e]:offsets[e + 1]] = True
    assert np.all(got[~inside] == NAN16), f"{what}: a row outside every group was written"
    if mode == "int":
        assert_bits_equal(got[inside], ref[inside], what)
    else:
        assert_close(got[inside], ref[inside], what)


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("b_layout", ["row", "col"])
@pytest.mark.parametrize("case", ["small_groups", "mid_groups", "large_groups"])
def test_grouped_parity(mode, b_layout, case):
    if case == "small_groups":      # 128 x 128 register-path tile
        sizes = np.array([0, 37, 130, 0, 1, 64, 255, 3])
        K, N = 100, 70
    elif case == "mid_groups":      # the same tile, with whole 16-byte B rows (N = 264)
        sizes = np.array([0, 37, 130, 0, 1, 64, 255, 3, 200])
        K, N = 160, 264
    else:                           # 256 x 256 LDS-DMA tile (groups average >= 256 rows)
        sizes = np.array([300, 0, 700, 517])
        K, N = 160, 264
    lead, tail = 3, 5
    offsets = np.concatenate([[lead], lead + np.cumsum(sizes)]).astype(np.int64)
    M = int(offsets[-1]) + tail
    G = len(sizes)
    A = synth.matrix(M, K, 12000 + K, 0, mode)
    Bs, b = experts(G, K, N, 12100 + K, mode, b_layout)
    ref = oracle.gemm_grouped(A, Bs, offsets, N, K, C=np.full((M, N), NAN16, dtype=np.uint16),
                              nthreads=ORACLE_THREADS)
    a = place(A, "row", (1, (-K) % 8 + 8))       # NaN after every row's K tail
    off = torch.from_numpy(offsets).to(DEV)
    outs = [run_grouped(a, b, off, Out(M, N)) for _ in range(2)]
    assert_bits_equal(outs[1], outs[0], f"grouped rerun {case}")
    check_groups(outs[0], ref, offsets, mode, f"grouped {case} {mode} B={b_layout}")


def test_grouped_shared_weight_is_the_plain_product():
    # ldb_g = 0: every group multiplies by the same B.
    M, K, N, G = 300, 64, 96, 5
    A = synth.matrix(M, K, 12200, 0, "int")
    B = synth.matrix(K, N, 12200, 1, "int")
    offsets = np.array([0, 10, 10, 150, 299, 300], dtype=np.int64)
    b = to_dev(B)[None].expand(G, K, N)
    assert b.stride(0) == 0
    got = run_grouped(to_dev(A), b, torch.from_numpy(offsets).to(DEV), Out(M, N))
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS)
    assert_bits_equal(got, ref, "grouped with one shared B")


def test_grouped_offsets_are_clamped():
    # Offsets outside [0, M] and a decreasing pair: nothing outside the view
    # changes (Out's canaries), and rows claimed by exactly one group are right.
    M, K, N = 40, 32, 24
    A = synth.matrix(M, K, 12300, 0, "int")
    Bs, b = experts(3, K, N, 12300, "int", "row")
    offsets = np.array([-10, 5, 3, M + 100], dtype=np.int64)
    got = run_grouped(to_dev(A), b, torch.from_numpy(offsets).to(DEV), Out(M, N))
    ref = oracle.gemm_grouped(A, Bs, [0, 5, 5, M], N, K)      # g1 empty after clamping
    assert_bits_equal(got[:3], ref[:3], "rows of group 0 only")
    ref2 = oracle.gemm_grouped(A, Bs, [0, 0, 0, M], N, K)
    assert_bits_equal(got[5:], ref2[5:], "rows of group 2 only")


def test_grouped_moe_shape_sampled():
    # The mixture-of-experts shape of the benchmark: 131072 routed tokens over
    # 32 experts (seeded skewed counts), K = 7168, N = 2048; sampled rows of
    # every group against the oracle.
    G, M, K, N = 32, 131072, 7168, 2048
    sizes = synth.group_sizes(G, M, 11)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    say("grouped MoE: generating inputs")
    a = to_dev(synth.matrix(M, K, 4001, 0))
    Bs, b = experts(G, K, N, 4101, "uniform", "row")
    off = torch.from_numpy(offsets).to(DEV)
    say("grouped MoE: launch")
    c = g.gemm_grouped(a, b, off)
    torch.cuda.synchronize()
    got = to_host(c)
    rng = np.random.default_rng(5)
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, 2)]))
        A_rows = synth.rows_of(rows, K, 4001, 0)
        ref = oracle.gemm(A_rows, (K, 1), Bs[e], (N, 1), len(rows), N, K, nthreads=ORACLE_THREADS)
        assert_close(got[rows], ref, f"MoE group {e} rows {rows.tolist()}")


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("case", ["small_groups", "mid_groups", "large_groups"])
def test_grouped_bf16_parity(mode, case):
    # gemm_bf16_grouped: the same launches with bfloat16 A, B and C.
    if case == "small_groups":
        sizes, K, N = np.array([0, 37, 130, 0, 1, 64, 255, 3]), 100, 70
    elif case == "mid_groups":
        sizes, K, N = np.array([0, 37, 130, 0, 1, 64, 255, 3, 200]), 160, 264
    else:
        sizes, K, N = np.array([300, 0, 700, 517]), 160, 264
    offsets = np.concatenate([[3], 3 + np.cumsum(sizes)]).astype(np.int64)
    M = int(offsets[-1]) + 5
    G = len(sizes)
    A = synth.matrix(M, K, 12500 + K, 0, mode, fmt="bf16")
    Bs = np.stack([synth.matrix(K, N, 12600 + K, 16 + e, mode, fmt="bf16") for e in range(G)])
    ref = oracle.gemm_grouped(A, Bs, offsets, N, K, C=np.full((M, N), NAN16, dtype=np.uint16),
                              nthreads=ORACLE_THREADS, dtype="bf16")
    a = place(A, "row", (1, (-K) % 8 + 8)).view(torch.bfloat16)
    b = to_dev(Bs).view(torch.bfloat16)
    off = torch.from_numpy(offsets).to(DEV)
    out = Out(M, N)
    out.view = out.view.view(torch.bfloat16)
    got = run_grouped(a, b, off, out)
    inside = np.zeros(M, dtype=bool)
    for e in range(G):
        inside[offsets[e]:offsets[e + 1]] = True
    assert np.all(got[~inside] == NAN16), "a row outside every group was written"
    if mode == "int":
        assert_bits_equal(got[inside], ref[inside], f"bf16 grouped {case}")
    else:
        assert_close_bf16(got[inside], ref[inside], f"bf16 grouped {case}")


F8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@pytest.mark.parametrize("b_layout", ["kcontig", "ncontig"])
@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("case", ["small_groups", "large_groups"])
def test_grouped_f8_parity(case, mode, b_layout):
    # gemm_f8_grouped: E4M3 A, E5M2 experts, fp16 C; rows padded with the
    # FP8 NaN byte 0x7F, which must never be read.
    fa, fb = "e4m3", "e5m2"
    if case == "small_groups":
        sizes, K, N = np.array([0, 37, 130, 0, 1, 64, 255, 3]), 100, 80
    else:
        sizes, K, N = np.array([300, 0, 700, 517]), 160, 272
    offsets = np.concatenate([[3], 3 + np.cumsum(sizes)]).astype(np.int64)
    M = int(offsets[-1]) + 5
    G = len(sizes)
    A = synth.matrix(M, K, 12700 + K, 0, mode, fmt=fa)
    Bs = np.stack([synth.matrix(K, N, 12800 + K, 16 + e, mode, fmt=fb) for e in range(G)])
    lda = K + (-K) % 16 + 16
    abuf = np.full((M, lda), 0x7F, dtype=np.uint8)
    abuf[:, :K] = A
    a = torch.from_numpy(abuf).to(DEV).view(F8_TORCH[fa])[:, :K]
    if b_layout == "kcontig":                   # each B_g stored [N, K]
        ld = K + (-K) % 16 + 16
        bbuf = np.full((G, N, ld), 0x7F, dtype=np.uint8)
        bbuf[:, :, :K] = Bs.transpose(0, 2, 1)
        b = torch.from_numpy(bbuf).to(DEV).view(F8_TORCH[fb])[:, :, :K].transpose(1, 2)
    else:                                       # each B_g stored [K, N]
        bbuf = np.full((G, K, N + 16), 0x7F, dtype=np.uint8)
        bbuf[:, :, :N] = Bs
        b = torch.from_numpy(bbuf).to(DEV).view(F8_TORCH[fb])[:, :, :N]
    ref = np.full((M, N), NAN16, dtype=np.uint16)
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            ref[r0:r1] = oracle.gemm(np.ascontiguousarray(A[r0:r1]), (K, 1), Bs[e], (N, 1), r1 - r0, N,
                                     K, dtype="f8", fmt_a=fa, fmt_b=fb, nthreads=ORACLE_THREADS)
    off = torch.from_numpy(offsets).to(DEV)
    got = run_grouped(a, b, off, Out(M, N))
    check_groups(got, ref, offsets, mode, f"f8 grouped {case} {mode} B={b_layout}")
