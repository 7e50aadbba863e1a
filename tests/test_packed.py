"""GPU parity of the pre-packed static B path (gemm_f16_pack_b +
gemm_f16_packed; the C500 log's weight packing done once, outside the timed
region) against the oracle, and against the general-stride path on integer
inputs.  B is packed from several layouts; padding of A rows is NaN.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, ORACLE_THREADS, Out, assert_bits_equal, assert_close, place, say,
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
