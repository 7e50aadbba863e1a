"""GPU parity of the bfloat16 entry points (gemm_bf16*) against the oracle's
bfloat16 product, on the same seeded logical values rounded to bfloat16.

Acceptance: bit-exact on integer inputs (every fp32 partial sum is an exact
integer, and both sides round the same exact sum once to bfloat16);
|C_gpu - C_oracle| <= 1e-2 + 8e-3 |C_oracle| on U(-1, 1) inputs (one
bfloat16 ulp is at most 2^-7 |C|).  The kernel families are forced as for
fp16: main (full-line-A and 128x128 tiles), split-K, skinny MFMA tiles and
the decode kernel (B N-contiguous, or as [N, K] rows).
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, ORACLE_THREADS, Out, assert_bits_equal, assert_close_bf16, place, say,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


def bdev(bits):
    return to_dev(bits).view(torch.bfloat16)


def bplace(bits, layout, pad=(0, 0)):
    return place(bits, layout, pad).view(torch.bfloat16)


class BOut(Out):
    """Out (NaN-filled view inside canaries) holding bfloat16 elements."""

    def __init__(self, M, N, ldc=None):
        super().__init__(M, N, ldc)
        self.view = self.view.view(torch.bfloat16)


def ref_bf16(A, B, rows=None):
    K, N = B.shape
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (N, 1), A.shape[0], N, K, nthreads=ORACLE_THREADS, dtype="bf16")


def run(a, b, out, **kw):
    say(f"bf16 gemm M={a.shape[0]} N={b.shape[1]} K={a.shape[1]} a.stride={a.stride()} "
        f"b.stride={b.stride()} opts={kw}")
    g.gemm(a, b, out=out.view, **kw)
    torch.cuda.synchronize()
    return out.result()


def check(got, ref, mode, what):
    if mode == "int":
        assert_bits_equal(got, ref, what)
    else:
        assert_close_bf16(got, ref, what)


VARIANTS = [dict(variant="auto"), dict(variant="main"), dict(variant="main", tile=14),
            dict(variant="main", tile=1), dict(variant="splitk", split_k=3),
            dict(variant="splitk", tile=14, split_k=2), dict(variant="main", tile=7),
            dict(variant="splitk", tile=7, split_k=2), dict(variant="main", tile=8)]


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_bf16_edge_130x70x65(mode, b_layout):
    M, N, K = 130, 70, 65
    A = synth.matrix(M, K, 1001, 0, mode, fmt="bf16")
    B = synth.matrix(K, N, 1001, 1, mode, fmt="bf16")
    ref = ref_bf16(A, B)
    a, b = bplace(A, "row", (1, 3)), bplace(B, b_layout, (1, 5))
    for kw in VARIANTS:
        check(run(a, b, BOut(M, N), **kw), ref, mode, f"bf16 edge {mode} B={b_layout} {kw}")


@pytest.mark.parametrize("n", [256, 1024])
def test_bf16_square(n):
    A = synth.matrix(n, n, 2000 + n, 0, fmt="bf16")
    B = synth.matrix(n, n, 2000 + n, 1, fmt="bf16")
    ref = ref_bf16(A, B)
    a, b = bdev(A), bdev(B)
    for kw in VARIANTS:
        check(run(a, b, BOut(n, n), **kw), ref, "uniform", f"bf16 square {n} {kw}")
    Bt = np.ascontiguousarray(B.T)
    bt = bdev(Bt).t()
    check(run(a, bt, BOut(n, n)), ref, "uniform", f"bf16 square {n} transposed B")


@pytest.mark.parametrize("b_layout", ["row", "col"])
@pytest.mark.parametrize("M", [1, 2, 4, 16, 64])
def test_bf16_skinny(M, b_layout):
    N, K = 2048, 7168
    A = synth.matrix(M, K, 3000 + M, 0, fmt="bf16")
    B = synth.matrix(K, N, 3000 + M, 1, fmt="bf16")
    ref = ref_bf16(A, B)
    a, b = bdev(A), bplace(B, b_layout)
    p = g.plan(a, b)
    assert p["variant"] == "skinny"
    for kw in (dict(variant="auto"), dict(variant="skinny", split_k=1),
               dict(variant="skinny", split_k=8), dict(variant="skinny", tile=3)):
        check(run(a, b, BOut(M, N), **kw), ref, "uniform", f"bf16 skinny M={M} B {b_layout} {kw}")
    Ai = synth.matrix(M, 128, 3100 + M, 0, "int", fmt="bf16")
    Bi = synth.matrix(128, N, 3100 + M, 1, "int", fmt="bf16")
    check(run(bdev(Ai), bplace(Bi, b_layout), BOut(M, N)), ref_bf16(Ai, Bi), "int",
          f"bf16 skinny int M={M} B {b_layout}")


def test_bf16_moe_shape_sampled():
    M, N, K = 131072, 2048, 7168
    say("bf16 MoE: generating inputs")
    A = synth.matrix(M, K, 4001, 0, fmt="bf16")
    B = synth.matrix(K, N, 4001, 1, fmt="bf16")
    a, b = bdev(A), bdev(B)
    assert g.plan(a, b)["tile_id"] == 14
    say("bf16 MoE: launch")
    c = g.gemm(a, b)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], rng.integers(0, M, 24)]))
    got = to_host(c.view(torch.float16))[rows]
    check(got, ref_bf16(A, B, rows), "uniform", "bf16 MoE sampled rows")
