"""GPU parity of the stream-K variant (TileLang tutorial ch. 14, section 4.2,
in the deterministic form of include/gemm_f16.h): whole waves of 256x256
tiles run as in the main variant, the tail tiles are split over K into fp32
partials, and a fixed-order fix-up sums them.  Acceptance as in test_parity:
bit-exact on integer inputs, the elementwise tolerance on U(-1, 1).  The
caller workspace is NaN-filled, so a fix-up read of a slot that no partial
wrote would show up as NaN.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
import synth
from gpu_util import (DEV, ORACLE_THREADS, Out, assert_bits_equal, assert_close, dev_nan, place,
                      say, to_dev, to_host)

pytestmark = pytest.mark.gpu


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def reference(A, B, rows=None):
    K, N = B.shape
    if rows is not None:
        A = np.ascontiguousarray(A[rows])
    return oracle.gemm(A, (K, 1), B, (N, 1), A.shape[0], N, K, nthreads=ORACLE_THREADS)


def run(a, b, out, **kw):
    p = g.plan(a, b, out=out.view, **kw)
    say(f"gemm M={a.shape[0]} N={b.shape[1]} K={a.shape[1]} b.stride={b.stride()} opts={kw} plan={p}")
    ws = dev_nan(p["workspace_bytes"] // 2 + 256)
    g.gemm(a, b, out=out.view, workspace=ws, **kw)
    torch.cuda.synchronize()
    return p, out.result()


@pytest.mark.parametrize("mode", ["int", "uniform"])
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_streamk_every_tile_in_the_tail(mode, b_layout):
    # 3 x 3 tiles, fewer than one wave: every tile is split; ragged M, N, K
    # (700 = ten 64-k super-steps and a 60-k tail).
    M, N, K = 600, 520, 700
    A = synth.matrix(M, K, 13000, 0, mode)
    B = synth.matrix(K, N, 13001, 1, mode)
    ref = reference(A, B)
    pad = (-K) % 8 + 8                  # K-contiguous rows stay 16-byte aligned; NaN past K
    a = place(A, "row", (1, pad))
    b = to_dev(B) if b_layout == "row" else place(B, "col", (1, pad))
    for s in (1, 3, 5):
        p, got = run(a, b, Out(M, N), variant="streamk", split_k=s)
        ks = -(-(-(-K // s)) // 64) * 64        # K ranges are whole 64-k super-steps
        assert (p["variant"], p["tile_id"], p["sk_tiles"], p["grid"], p["split_k"]) == \
            ("streamk", 14, 9, 0, -(-K // ks))
        what = f"stream-K {M}x{N}x{K} {mode} B={b_layout} S={s}"
        if mode == "int":
            assert_bits_equal(got, ref, what)
        else:
            assert_close(got, ref, what)


def test_streamk_tail_after_a_whole_wave():
    # 18 x 17 = 306 tiles: one whole wave on the main kernel, the remaining
    # 306 - cus tiles split three ways; ragged edges on both axes.
    M, N, K = 4389, 4136, 481
    W = cus()
    A = synth.matrix(M, K, 13100, 0, "int")
    B = synth.matrix(K, N, 13101, 1, "int")
    a, b = place(A, "row", (1, (-K) % 8 + 8)), to_dev(B)
    p, got = run(a, b, Out(M, N), variant="streamk", split_k=3)
    T = 18 * 17
    assert (p["sk_tiles"], p["grid"], p["split_k"]) == (T % W, T - T % W, 3)
    ref = reference(A, B)
    assert_bits_equal(got, ref, "stream-K tail after one wave")
    _, again = run(a, b, Out(M, N), variant="streamk", split_k=3)
    assert_bits_equal(again, got, "stream-K rerun")


def test_streamk_auto_choice_matches_main():
    # 17 x 16 = 272 tiles with K = 2048: a final wave of 16 tiles is at most
    # half full, so the automatic plan takes the stream-K tail.  Integer sums
    # are exact in fp32, so it must agree bit for bit with the main plan;
    # sampled rows, including the last tile row, against the oracle.
    M, N, K = 4352, 4096, 2048
    W = cus()
    A = synth.matrix(M, K, 13200, 0, "int")
    B = synth.matrix(K, N, 13201, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    T = 17 * 16
    if T % W == 0 or 2 * (T % W) > W:
        pytest.skip(f"{W} compute units: no half-empty final wave for this shape")
    assert p["variant"] == "streamk" and p["sk_tiles"] == T % W
    say(f"stream-K auto plan {p}")
    got = to_host(g.gemm(a, b))
    main = to_host(g.gemm(a, b, variant="main"))
    torch.cuda.synchronize()
    assert_bits_equal(got, main, "stream-K auto vs main")
    rows = np.array([0, 1, 255, 2000, 4095, 4096, 4351])
    assert_bits_equal(got[rows], reference(A, B, rows), "stream-K auto sampled rows")


def test_streamk_bf16():
    M, N, K = 600, 520, 700
    A = synth.matrix(M, K, 13300, 0, "int", fmt="bf16")
    B = synth.matrix(K, N, 13301, 1, "int", fmt="bf16")
    ref = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, nthreads=ORACLE_THREADS, dtype="bf16")
    pad = (-K) % 8 + 8                  # 16-byte aligned rows, bfloat16 NaN past K
    Ap = np.pad(A, ((0, 0), (0, pad)), constant_values=0x7FC0)
    a = torch.from_numpy(Ap.view(np.int16)).to(DEV).view(torch.bfloat16)[:, :K]
    b = torch.from_numpy(B.view(np.int16)).to(DEV).view(torch.bfloat16)
    say("stream-K bf16 600x520x700")
    c = g.gemm(a, b, variant="streamk", split_k=4)
    torch.cuda.synchronize()
    got = c.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bits_equal(got, ref, "stream-K bf16 integer inputs")


def test_streamk_auto_small_grid():
    # 6 x 6 = 36 tiles of 256 x 256, under half a wave, with a long K: the
    # automatic plan sends every tile to the stream-K tail rather than to the
    # 128 x 128 tile.  Integer inputs keep every fp32 sum exact (|sum| <= 16 K
    # < 2^24), so the result must equal the main plan's and the oracle's bit
    # for bit; sampled rows against the oracle, including the last tile row.
    M, N, K = 1536, 1536, 8192
    W = cus()
    A = synth.matrix(M, K, 13400, 0, "int")
    B = synth.matrix(K, N, 13401, 1, "int")
    a, b = to_dev(A), to_dev(B)
    p = g.plan(a, b)
    if 2 * 36 >= W:
        pytest.skip(f"{W} compute units: 36 tiles are at least half a wave")
    assert (p["variant"], p["tile_id"], p["sk_tiles"], p["grid"]) == ("streamk", 14, 36, 0), p
    say(f"stream-K small-grid auto plan {p}")
    got = to_host(g.gemm(a, b))
    main = to_host(g.gemm(a, b, variant="main", tile=1))
    torch.cuda.synchronize()
    assert_bits_equal(got, main, "stream-K small grid vs 128x128 main")
    rows = np.array([0, 1, 255, 256, 777, 1279, 1280, 1535])
    assert_bits_equal(got[rows], reference(A, B, rows), "stream-K small grid sampled rows")
