"""gemm_f16_noalloc (the entry point for callers that cannot allocate) through
the C-ABI, against gemm_f16_ex on the same inputs: its plans are the
automatic plans without a packing pass, run on the same kernels, with the
workspace in the library's fixed per-GPU scratch array instead of a caller's
or an allocated one.  Two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents), then a plan too large for the
scratch, which must be refused before anything runs.  Acceptance as for the
other parity tests: bit-exact on integer inputs, the elementwise tolerance
on U(-1, 1) inputs (the plans being the same, the bits match there too)."""
import ctypes

import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
from dense_tiled_gemm_fp16_amd import _lib
import synth
from gpu_util import Out, assert_bits_equal, assert_close, say, to_dev

pytestmark = pytest.mark.gpu


def call_noalloc(a, b, out):
    M, K = a.shape
    N = b.shape[1]
    rc = g.lib.gemm_f16_noalloc(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
                                b.stride(1), out.data_ptr(), out.stride(0), M, N, K,
                                torch.cuda.current_stream().cuda_stream)
    return rc


def call_ex(a, b, out):
    M, K = a.shape
    N = b.shape[1]
    return g.lib.gemm_f16_ex(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
                             b.stride(1), out.data_ptr(), out.stride(0), M, N, K,
                             torch.cuda.current_stream().cuda_stream, None, 0, None)


def pair(M, N, K, seed, mode):
    A = synth.matrix(M, K, seed, 0, mode)
    B = synth.matrix(K, N, seed, 1, mode)
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    say(f"noalloc {mode} {M}x{N}x{K} plan {p}")
    assert 0 < p["workspace_bytes"] <= _lib.SCRATCH_BYTES, p    # the case uses the scratch
    o1, o2 = Out(M, N), Out(M, N)
    assert call_noalloc(a, b, o1.view) == 0
    assert call_ex(a, b, o2.view) == 0
    torch.cuda.synchronize()
    got, ref = o1.result(), o2.result()
    if mode == "int":
        assert_bits_equal(got, ref, f"noalloc {M}x{N}x{K}")
    else:
        assert_close(got, ref, f"noalloc {M}x{N}x{K}")
        assert_bits_equal(got, ref, f"noalloc {M}x{N}x{K} (same plan, same bits)")


@pytest.mark.parametrize("mode", ["uniform", "int"])
def test_noalloc_two_calls_then_smaller(mode):
    pair(384, 384, 16384 if mode == "uniform" else 4096, 33001, mode)   # split-K partials
    pair(1, 2048, 7168 if mode == "uniform" else 1024, 33002, mode)     # decode partials


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    M = N = 2048                 # stream-K, all 64 tiles in 4 K ranges: 64 MiB of partials
    K = 8192
    a = torch.zeros((M, K), dtype=torch.float16, device="cuda:0")
    b = torch.zeros((K, N), dtype=torch.float16, device="cuda:0")
    p = g.plan(a, b)
    assert p["workspace_bytes"] > _lib.SCRATCH_BYTES, p
    out = Out(M, N)
    say(f"noalloc refusal {M}x{N}x{K} plan {p}")
    assert call_noalloc(a, b, out.view) == -10
    torch.cuda.synchronize()
    assert np.all(out.result() == 0x7E00)        # nothing ran: C untouched
    with pytest.raises(g.GemmError):
        g.gemm_noalloc(a, b, out.view)
