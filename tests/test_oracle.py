"""Pins of the CPU oracle to things other than itself: the pages' worked
examples (tests/golden), IEEE 754 special cases, numpy's binary16 conversion,
exact integer and rational arithmetic, and textbook special cases."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import model


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def val(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- codec

def test_decode_all_patterns_matches_numpy_and_roundtrips():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 1023
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    back = oracle.f64_to_f16(got)
    assert np.array_equal(back[~nan], bits[~nan])
    assert np.all(np.isnan(val(back[nan])))


def test_encode_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(12345)
    n = 1_000_000
    x = rng.standard_normal(n) * 10.0 ** rng.uniform(-9, 5.5, n)
    x = np.concatenate([x, [0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 1e300,
                            2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 5e-324]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16(x), ref)


def test_encode_every_midpoint_ties_to_even():
    lo = np.arange(0, 0x7BFF, dtype=np.uint16)           # finite, positive, below max
    mid = (val(lo) + val(lo + 1)) / 2.0                    # exact in binary64
    for sgn in (1.0, -1.0):
        got = oracle.f64_to_f16(sgn * mid)
        assert np.array_equal(got, (sgn * mid).astype(np.float16).view(np.uint16))
        assert np.all(got & 1 == 0)                       # the even neighbour
    # half-way between the largest finite value and 2^16 overflows to infinity
    assert oracle.f64_to_f16(np.array([65520.0, -65520.0])).tolist() == [0x7C00, 0xFC00]


# ---------------------------------------------------------------- rounding of the product

def _one(a, b, K):
    A = f16(np.array(a, dtype=np.float64).reshape(1, K))
    B = f16(np.array(b, dtype=np.float64).reshape(K, 1))
    return int(oracle.gemm(A, (K, 1), B, (1, 1), 1, 1, K)[0, 0])


def test_final_rounding_is_ties_to_even_with_overflow_to_inf():
    # 1 + 3*2^-11 lies half-way between 0x3C01 and 0x3C02: RNE picks 0x3C02
    # (round toward zero would give 0x3C01).
    assert _one([1.0, 3 * 2.0 ** -11], [1.0, 1.0], 2) == 0x3C02
    # 1 + 2^-11 lies half-way between 0x3C00 and 0x3C01: RNE picks 0x3C00
    # (round half away from zero would give 0x3C01).
    assert _one([1.0, 2.0 ** -11], [1.0, 1.0], 2) == 0x3C00
    # 256 * 256 = 65536 overflows binary16: +inf (round toward zero gives 0x7BFF)
    assert _one([256.0], [256.0], 1) == 0x7C00
    assert _one([65504.0, 16.0], [1.0, 1.0], 2) == 0x7C00    # 65520, the overflow tie
    assert _one([65504.0, 8.0], [1.0, 1.0], 2) == 0x7BFF     # 65512 rounds down
    # a sum that cancels to zero is +0, not -0
    assert _one([1.0, -1.0], [1.0, 1.0], 2) == 0x0000


# ---------------------------------------------------------------- the pages' worked examples

def test_k3_block_masking_example(gold):
    g = gold("k3_masking.txt")
    a, b = [g["a"]], [[v] for v in g["b"]]
    zero = model.tiled_gemm(a, b, 1, 1, g["block"], k_policy="mask")
    wrong = model.tiled_gemm(a, b, 1, 1, g["block"], k_policy="modulo")
    assert zero.C[0][0] == g["expected_zero_fill"]
    assert wrong.C[0][0] == g["expected_modulo"]
    assert zero.last_round_valid_k == 1
    assert val(_one(g["a"], g["b"], 3)) == g["expected_zero_fill"]


def test_stride_example(gold):
    g = gold("stride_example.txt")
    buf = f16(g["buffer"])
    (K, N), (sk, sn) = g["shape"], g["stride"]
    e1 = f16([[0.0, 1.0, 0.0]])                       # selects row 1 of B
    right = val(oracle.gemm(e1, (K, 1), buf, (sk, sn), 1, N, K))[0]
    wk, wn = g["wrong_stride"]
    wrong = val(oracle.gemm(e1, (K, 1), buf, (wk, wn), 1, N, K))[0]
    assert right[0] == g["b10"] and wrong[0] == g["b10_wrong"]
    # The whole row follows from the same two stride rules: [11, 21] vs [12, 20].
    assert right.tolist() == [11.0, 21.0] and wrong.tolist() == [12.0, 20.0]


def test_int64_offsets(gold):
    g = gold("int64_offset.txt")
    assert g["row"] * g["stride"] == g["offset"]
    with np.errstate(over="ignore"):
        wrapped = np.array([g["row"]], np.int32) * np.array([g["stride"]], np.int32)
    assert int(wrapped[0]) == g["offset_int32"]
    # A sparse 8 GiB buffer (only two pages are ever touched): element 0 and
    # element 2^32 hold different values; row 65536 with row stride 65536 must
    # read the second one.
    A = np.zeros(g["offset"] + 1, dtype=np.uint16)
    A[0] = f16(1.0)
    A[g["offset"]] = f16(2.0)
    B = f16([[3.0]])
    out = oracle.gemm_points(A, (g["stride"], 1), B, (1, 1), 1, [0, g["row"]], [0, 0])
    assert val(out).tolist() == [3.0, 6.0]


def test_read_ledger_4x4(gold):
    g = gold("read_ledger_4x4.txt")
    M, N, K = g["M"], g["N"], g["K"]
    A = [[(3 * i + 5 * k) % 7 - 3 for k in range(K)] for i in range(M)]
    B = [[(2 * k - j) % 5 - 2 for j in range(N)] for k in range(K)]
    exact = (np.array(A, dtype=np.int64) @ np.array(B, dtype=np.int64)).tolist()
    naive = model.tiled_gemm(A, B, 1, 1, K)
    tiles = model.tiled_gemm(A, B, 2, 2, 2)
    whole = model.tiled_gemm(A, B, 4, 4, 4)
    assert model.naive_reads(M, N, K) == naive.reads == g["naive_reads"]
    assert naive.writes == g["naive_writes"]
    assert tiles.reads == g["tile2x2_reads"]
    assert whole.reads == g["whole_reads"]
    for run in (naive, tiles, whole):
        assert run.C == exact
    # the tutorial's general re-read formula b*MNK*(1/m1 + 1/n1) with b = 1
    for (m1, n1), reads in (((1, 1), 128), ((2, 2), 64), ((4, 4), 32)):
        assert model.tile_reread_bytes(M, N, K, m1, n1, 1) == reads


def test_edge_geometry_130x70x65(gold):
    g = gold("geometry_130x70x65.txt")
    M, N, K = g["M"], g["N"], g["K"]
    A = synth.matrix(M, K, seed=1002, tensor=0, mode="int")
    B = synth.matrix(K, N, seed=1002, tensor=1, mode="int")
    Ai, Bi = val(A).astype(np.int64), val(B).astype(np.int64)
    run = model.tiled_gemm(Ai.tolist(), Bi.tolist(), g["BM"], g["BN"], g["BK"])
    assert list(run.grid) == g["grid"] and run.k_rounds == g["k_rounds"]
    corner = len(run.valid_outputs) - 1
    assert run.valid_outputs[corner] == g["corner_valid_outputs"] \
        == g["corner_valid_rows"] * g["corner_valid_cols"]
    assert run.last_round_valid_k == g["last_round_valid_k"]
    useful = model.flops(M, N, K) / run.block_flops
    assert model.flops(M, N, K) == 1_183_000 and run.block_flops == 3_538_944
    assert round(100 * useful, 1) == g["useful_percent"]
    # the tiled method, the exact integer product and the oracle all agree
    exact = Ai @ Bi
    assert run.C == exact.tolist()
    assert np.array_equal(val(oracle.gemm(A, (K, 1), B, (N, 1), M, N, K)), exact)
    # wrapping M/N indices is harmless (invalid rows/columns are never stored),
    # wrapping K is not
    assert model.tiled_gemm(Ai.tolist(), Bi.tolist(), 64, 32, 32, mn_policy="modulo").C == run.C
    assert model.tiled_gemm(Ai.tolist(), Bi.tolist(), 64, 32, 32, k_policy="modulo").C != run.C


def test_ledger_closed_forms(gold):
    g = gold("ledger_closed_forms.txt")
    assert model.min_bytes(4096, 4096, 4096, 2) == g["min_bytes_4096_mib"] * 2 ** 20
    naive = model.tile_reread_bytes(4096, 4096, 4096, 1, 1, 2)
    assert naive == 2 * 4096 ** 3 * 2 and round(float(naive) / 1e9) == g["naive_bytes_4096_gb"]
    assert model.stage_bytes(128, 128, 32, 2) == g["stage_bytes_128x128x32"]
    assert model.stage_bytes(128, 128, 32, 2, stages=3) == g["stage_bytes_3_stages"]
    assert model.stage_intensity(64, 64, 2) == g["i_stage_64"]
    assert model.stage_intensity(128, 128, 2) == g["i_stage_128"]
    assert model.accumulator_bytes(64, 64) == g["acc_bytes_64"]
    assert model.accumulator_bytes(128, 128) == g["acc_bytes_128"]
    for m in (256, 1024, 4096):
        assert model.intensity(m, m, m, 2) == Fraction(2 * m, 3 * 2)


# ---------------------------------------------------------------- brute force and special cases

def _views(M, N, K, seed):
    """The same logical integer A[M,K] and B[K,N] in four storage layouts,
    each as (buffer, offset, strides).  Padding is NaN so a read outside
    the view poisons the result."""
    nan = np.uint16(0x7E00)
    A = synth.matrix(M, K, seed, 0, mode="int")
    B = synth.matrix(K, N, seed, 1, mode="int")
    out = []
    out.append(((A.ravel(), 0, (K, 1)), (B.ravel(), 0, (N, 1))))
    out.append(((np.ascontiguousarray(A.T).ravel(), 0, (1, M)),
                (np.ascontiguousarray(B.T).ravel(), 0, (1, K))))
    # padded slices with offsets
    pa = np.full((M + 2, K + 3), nan, np.uint16)
    pa[1:M + 1, 2:K + 2] = A
    pb = np.full((K + 1, N + 5), nan, np.uint16)
    pb[1:, 3:N + 3] = B
    out.append(((pa.ravel(), 1 * (K + 3) + 2, (K + 3, 1)), (pb.ravel(), (N + 5) + 3, (N + 5, 1))))
    # column-strided views (every other element)
    sa = np.full((M, 2 * K), nan, np.uint16)
    sa[:, ::2] = A
    sb = np.full((2 * K, N), nan, np.uint16)
    sb[::2, :] = B
    out.append(((sa.ravel(), 0, (2 * K, 2)), (sb.ravel(), 0, (2 * N, 1))))
    exact = val(A).astype(np.int64) @ val(B).astype(np.int64)
    return out, exact


def test_brute_force_tiny_shapes_exact():
    for M, N, K in itertools.product(range(1, 9), repeat=3):
        views, exact = _views(M, N, K, seed=M * 100 + N * 10 + K)
        for (abuf, aoff, lda), (bbuf, boff, ldb) in views:
            C = oracle.gemm(abuf, lda, bbuf, ldb, M, N, K, a_off=aoff, b_off=boff, nthreads=1)
            assert np.array_equal(val(C), exact), (M, N, K, lda, ldb)


def test_output_row_stride_and_untouched_padding():
    M, N, K = 5, 7, 9
    A = synth.matrix(M, K, 3, 0, mode="int")
    B = synth.matrix(K, N, 3, 1, mode="int")
    C = np.full(3 + M * 11, 0xABCD, dtype=np.uint16)
    oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, C=C, ldc=11, c_off=3)
    exact = val(A).astype(np.int64) @ val(B).astype(np.int64)
    view = C[3:].reshape(M, 11)
    assert np.array_equal(val(view[:, :N]), exact)
    assert np.all(view[:, N:] == 0xABCD) and np.all(C[:3] == 0xABCD)


def _frac_to_f16(v):
    """Exact nearest binary16 (ties to even) of a Fraction, by comparing the
    exact distances to the neighbours of a first guess."""
    g = np.float16(float(v))
    cand = {g, np.nextafter(g, np.float16(np.inf)), np.nextafter(g, np.float16(-np.inf))}
    best = sorted(cand, key=lambda c: (abs(Fraction(float(c)) - v),
                                       int(np.array(c).view(np.uint16)) & 1))
    return int(np.array(best[0]).view(np.uint16))


def test_uniform_inputs_against_exact_rational_sum():
    M, N, K = 12, 10, 700
    A = synth.matrix(M, K, 9, 0)
    B = synth.matrix(K, N, 9, 1)
    C, S = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, exact=True)
    # every U(-1,1) fp16 value is an integer multiple of 2^-24
    ai = (val(A) * 2.0 ** 24).astype(np.int64)
    bi = (val(B) * 2.0 ** 24).astype(np.int64)
    for i in range(M):
        for j in range(N):
            s = sum(int(x) * int(y) for x, y in zip(ai[i], bi[:, j]))
            exact = Fraction(s, 2 ** 48)
            bound = K * 2.0 ** -53 * float(np.sum(np.abs(val(A[i]) * val(B[:, j]))))
            assert abs(Fraction(S[i, j]) - exact) <= Fraction(bound)
            assert int(C[i, j]) == _frac_to_f16(exact), (i, j)


def test_matches_literal_python_loop():
    M, N, K = 7, 9, 13
    A = synth.matrix(M, K, 11, 0)
    B = synth.matrix(K, N, 11, 1)
    a, b = val(A), val(B)
    C = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K)
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(a[i, k]) * float(b[k, j])
            assert int(C[i, j]) == int(np.float64(s).astype(np.float16).view(np.uint16))


def test_identity_permutation_and_unit_row():
    M, K = 37, 29
    A = synth.matrix(M, K, 5, 0)
    eye = f16(np.eye(K))
    assert np.array_equal(oracle.gemm(A, (K, 1), eye, (K, 1), M, K, K), A)
    perm = np.random.default_rng(0).permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0                          # column j picks A[:, perm[j]]
    assert np.array_equal(oracle.gemm(A, (K, 1), f16(P), (K, 1), M, K, K), A[:, perm])
    B = synth.matrix(K, 23, 5, 1)
    e = np.zeros((1, K))
    e[0, 17] = 1.0
    assert np.array_equal(oracle.gemm(f16(e), (K, 1), B, (23, 1), 1, 23, K)[0], B[17])


def test_points_match_full_product():
    M, N, K = 33, 41, 57
    A = synth.matrix(M, K, 8, 0)
    Bt = synth.matrix(K, N, 8, 1, order="col")            # B as a transposed view
    full = oracle.gemm(A, (K, 1), Bt, (1, K), M, N, K)
    rng = np.random.default_rng(3)
    ii, jj = rng.integers(0, M, 200), rng.integers(0, N, 200)
    assert np.array_equal(oracle.gemm_points(A, (K, 1), Bt, (1, K), K, ii, jj), full[ii, jj])


def test_rejects_views_past_their_buffer():
    A = np.zeros(10, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(A, (5, 1), A, (1, 1), 3, 1, 5)
    with pytest.raises(ValueError):
        oracle.gemm(A, (5, 1), A, (1, 1), 0, 1, 5)


# ---------------------------------------------------------------- grouped product

def test_grouped_single_group_is_the_plain_product():
    A = synth.matrix(37, 19, 51, 0)
    B = synth.matrix(19, 23, 51, 1)
    got = oracle.gemm_grouped(A, B[None], [0, 37], 23, 19)
    assert np.array_equal(got, oracle.gemm(A, (19, 1), B, (23, 1), 37, 23, 19))


def test_grouped_brute_force_exact_integers():
    # Per group, every output equals the exact integer dot product with that
    # group's own B; rows outside the groups keep their prior value.
    rng = np.random.default_rng(7)
    for trial in range(20):
        G = int(rng.integers(1, 6))
        sizes = rng.integers(0, 5, G)
        lead, tail = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        M = lead + int(sizes.sum()) + tail
        if M == 0:
            continue
        N, K = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        offsets = np.concatenate([[lead], lead + np.cumsum(sizes)])
        Ai = rng.integers(-4, 5, (M, K))
        Bi = rng.integers(-4, 5, (G, K, N))
        C0 = np.full((M, N), 0x7E00, dtype=np.uint16)      # a NaN canary
        got = oracle.gemm_grouped(f16(Ai), f16(Bi), offsets, N, K, C=C0.copy())
        for r in range(M):
            g = [h for h in range(G) if offsets[h] <= r < offsets[h + 1]]
            if not g:
                assert np.array_equal(got[r], C0[r])
                continue
            want = [sum(int(Ai[r, k]) * int(Bi[g[0], k, j]) for k in range(K)) for j in range(N)]
            assert val(got[r]).tolist() == want


def test_grouped_rejects_bad_offsets():
    A = synth.matrix(4, 3, 1, 0)
    B = synth.matrix(3, 2, 1, 1)[None]
    for bad in ([0, 5], [-1, 3], [3, 2]):
        with pytest.raises(ValueError):
            oracle.gemm_grouped(A, B, bad, 2, 3)


# ---------------------------------------------------------------- bfloat16

def _torch_bf16_from_f32(x):
    """float32 values -> bfloat16 bits by torch (ties to even; a single
    rounding, since the inputs are exact in float32)."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    with np.errstate(invalid="ignore"):       # signalling NaN patterns
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    back = oracle.f64_to_bf16(got)
    assert np.array_equal(back[~nan], bits[~nan])


def test_bf16_encode_matches_torch_on_float32_values():
    rng = np.random.default_rng(99)
    x = (rng.standard_normal(500_000) * 10.0 ** rng.uniform(-40, 38, 500_000)).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40, 1.1e-38])])
    assert np.array_equal(oracle.f64_to_bf16(x.astype(np.float64)), _torch_bf16_from_f32(x))


def test_bf16_every_midpoint_ties_to_even():
    lo = np.arange(0, 0x7F7F, dtype=np.uint16)
    mid = (oracle.bf16_to_f64(lo) + oracle.bf16_to_f64(lo + 1)) / 2.0
    got = oracle.f64_to_bf16(mid)
    assert np.all(got & 1 == 0)
    assert np.array_equal(got, _torch_bf16_from_f32(mid.astype(np.float32)))


def test_bf16_closed_forms():
    cases = {
        1 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,   # above the midpoint: up (via float32 it would tie to 1.0)
        1 + 2.0 ** -8: 0x3F80,                # the midpoint itself: to even
        1 + 3 * 2.0 ** -8: 0x3F82,            # midpoint between 0x3F81 and 0x3F82: to even
        2.0 ** 128 * (1 - 2.0 ** -9): 0x7F80,  # halfway to 2^128: overflows to infinity
        2.0 ** 128 * (1 - 2.0 ** -8): 0x7F7F,  # the largest finite value
        2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000, 3 * 2.0 ** -134: 0x0002,
        -(2.0 ** -126): 0x8080,
    }
    got = oracle.f64_to_bf16(np.array(list(cases)))
    assert got.tolist() == list(cases.values())


def test_bf16_brute_force_small_products():
    # Integer inputs: each output is the exact integer sum rounded once to
    # bfloat16 (torch's float32 -> bfloat16 on the exact sum).
    rng = np.random.default_rng(3)
    for M, N, K in itertools.product((1, 3, 8), (1, 5), (1, 4, 9, 40)):
        Ai = rng.integers(-4, 5, (M, K))
        Bi = rng.integers(-4, 5, (K, N))
        A = _torch_bf16_from_f32(Ai)
        B = _torch_bf16_from_f32(Bi)
        got = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, dtype="bf16")
        assert np.array_equal(got, _torch_bf16_from_f32(Ai @ Bi))


# ------------------------------------------------------------------ FP8 inputs
# TileLang tutorial ch. 14, section 5 (low precision): FP8 operands in the
# E4M3 and E5M2 formats with wider accumulation.  The decoders are pinned to
# torch's float8 types (another implementation of the OCP definitions) on
# all 256 patterns, to closed forms, and the products to exact sums.

def _torch_f8(fmt):
    import torch
    return torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_f8_decode_all_patterns_matches_torch(fmt):
    import torch
    bits = np.arange(256, dtype=np.uint8)
    got = oracle.f8_to_f64(bits, fmt)
    ref = torch.from_numpy(bits).view(_torch_f8(fmt)).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f8_closed_forms():
    e4 = oracle.f8_to_f64(np.array([0x7E, 0x01, 0x08, 0x38, 0x7F, 0xFF, 0x80, 0x44], np.uint8), "e4m3")
    assert e4[0] == 448.0 and e4[1] == 2.0 ** -9 and e4[2] == 2.0 ** -6 and e4[3] == 1.0
    assert np.isnan(e4[4]) and np.isnan(e4[5]) and e4[6] == 0.0 and np.signbit(e4[6])
    assert e4[7] == 3.0
    e5 = oracle.f8_to_f64(np.array([0x7B, 0x01, 0x04, 0x3C, 0x7C, 0xFC, 0x7D, 0x3E], np.uint8), "e5m2")
    assert e5[0] == 57344.0 and e5[1] == 2.0 ** -16 and e5[2] == 2.0 ** -14 and e5[3] == 1.0
    assert e5[4] == np.inf and e5[5] == -np.inf and np.isnan(e5[6]) and e5[7] == 1.5


def _fraction_to_f16_bits(x):
    """Exact rational -> binary16 bits, ties to even (written from the format:
    quantum 2^(e-10) for 2^e <= |x| < 2^(e+1), e >= -14; overflow to inf)."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -14) - 10)
    m, r = divmod(a, q)
    m = int(m)
    if r > q / 2 or (r == q / 2 and m % 2 == 1):
        m += 1
    v = m * q
    if v >= 65520:
        return sign | 0x7C00
    if v < Fraction(2) ** -14:
        return sign | int(v / Fraction(2) ** -24)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    return sign | ((e + 15) << 10) | int(v / Fraction(2) ** (e - 10) - 1024)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
                                   ("e5m2", "e5m2")])
def test_f8_brute_force_exact_sums(fa, fb):
    # Random FP8 operands (finite patterns), each output the exact rational sum
    # rounded once to binary16; mixed formats decode each operand by its own.
    rng = np.random.default_rng(17)
    for M, N, K in itertools.product((1, 3), (1, 4), (1, 5, 33)):
        A = rng.integers(0, 256, (M, K)).astype(np.uint8)
        B = rng.integers(0, 256, (K, N)).astype(np.uint8)
        av, bv = oracle.f8_to_f64(A, fa), oracle.f8_to_f64(B, fb)
        A[~np.isfinite(av)] = 0
        B[~np.isfinite(bv)] = 0
        av, bv = oracle.f8_to_f64(A, fa), oracle.f8_to_f64(B, fb)
        got = oracle.gemm(A, (K, 1), B, (N, 1), M, N, K, dtype="f8", fmt_a=fa, fmt_b=fb)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(av[i, k]) * Fraction(bv[k, j]) for k in range(K))
                assert got[i, j] == _fraction_to_f16_bits(s), (i, j, float(s))


def test_f8_integer_product_equals_the_f16_product():
    # Integers in [-4, 4] are exact in both FP8 formats and in binary16, so the
    # FP8 product must equal the binary16 product of the same values.
    for fmt in ("e4m3", "e5m2"):
        A8 = synth.matrix(40, 70, 5, 0, "int", fmt=fmt)
        B8 = synth.matrix(70, 30, 5, 1, "int", fmt=fmt)
        A16 = oracle.f64_to_f16(oracle.f8_to_f64(A8, fmt))
        B16 = oracle.f64_to_f16(oracle.f8_to_f64(B8, fmt))
        want = oracle.gemm(A16, (70, 1), B16, (30, 1), 40, 30, 70)
        got = oracle.gemm(A8, (70, 1), B8, (30, 1), 40, 30, 70, dtype="f8", fmt_a=fmt, fmt_b=fmt)
        assert np.array_equal(got, want)
        pts = oracle.gemm_points(A8, (70, 1), B8, (30, 1), 70, [0, 39, 7], [0, 29, 11], dtype="f8",
                                 fmt_a=fmt, fmt_b=fmt)
        assert pts.tolist() == [want[0, 0], want[39, 29], want[7, 11]]
