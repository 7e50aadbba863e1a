"""GPU pin of the output rounding, on every output path of the library.

The final conversion of the fp32 sum to the output format is round to
nearest with ties to even, and a sum past the largest finite binary16 value
(65504) by half a step or more becomes infinity (the Triton article, section
"expose errors before comparing speed", asks for this last rounding to be
watched on its own; IEEE 754 fixes what it is).  The other parity tests use
sums that fp16 holds exactly or tolerances of a few units, so a kernel that
truncated or saturated would still pass them.  Here the inputs are
integers whose products and partial sums are exact in fp32 in any order, so
every kernel's fp32 sum equals the exact sum, and the exact sums are spread
over the binades [2^11, 2^16) where fp16 must round them (and, for bfloat16
output, over [2^8, 2^17)).  The output must then equal the oracle's bit for
bit.  Each case also plants one row of A and four columns of B whose sums are
exactly 65504, 65512, 65520 and 65528 (and their negatives): the oracle gives
0x7BFF, 0x7BFF, 0x7C00 and 0x7C00 for them, and so must every path.

Before comparing, each case asserts on the oracle's exact sums that it holds
enough rounded outputs and exact ties to tell round-to-nearest-even from
truncation and from rounding ties away from zero.

Paths: the 256x256 LDS-DMA tiles (ids 14 and 13) with N- and K-contiguous
B, the 256x256 and 128x128 register tiles, the pages' 64x32x32 tile, split-K
(256x256 and 128x128 partials, the fixed-order reduction at 1, 4 and 16
lanes per output), stream-K (its fix-up), the skinny MFMA tiles (16, 32 and 64
rows), the decode kernel (M <= 64 with N-contiguous B, M <= 16 with K-contiguous B), the pre-packed B, grouped products,
and the same in bfloat16 and FP8 (E4M3 and E5M2 operands, fp16 output).
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_fp16_amd as g
import oracle
from gpu_util import DEV, NAN16, ORACLE_THREADS, Out, assert_bits_equal, say, to_host

pytestmark = pytest.mark.gpu

E5M2_INTS = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16])
TORCH_FMT = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
             "e5m2": torch.float8_e5m2}

# (sum of B over the first K-1 rows, B in the last row): with the planted row
# of A (16 everywhere, 8 in the last k) the sums are 65520, 65512, 65504, 65528.
PLANTED = [(4095, 0), (4094, 1), (4094, 0), (4095, 1)]
PLANTED_BITS = [0x7C00, 0x7BFF, 0x7BFF, 0x7C00]


def to_format(vals, fmt):
    """Exact integer values -> bit patterns of the format (every value used is
    representable, so any correct encoder gives the same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(TORCH_FMT[fmt])
    if fmt in ("e4m3", "e5m2"):
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def column_with_sum(K, total, last, fmt):
    """A column of K integers in [0, 16]: the first K-1 sum to `total`, the
    last is `last`; values representable in the format."""
    col = np.zeros(K, dtype=np.int64)
    rest, k = total, 0
    while rest > 0:
        v = min(16, rest)
        if fmt == "e5m2" and v not in E5M2_INTS:
            v -= 1
        col[k] = v
        rest -= v
        k += 1
    assert k < K - 1, "K too short for the planted sum"
    col[K - 1] = last
    return col


def int_inputs(M, N, K, seed, fmt="f16", row_scales=(4, 8, 16), col_scales=(2, 4, 8, 16),
               plant=None):
    """Integer A [M, K] and B [K, N] (int64).  Row i of A is drawn from
    [0, r_i] (one row in eight from [-r_i, r_i], and about half the rows
    negated); column j of B from [0, c_j].  `plant` = (i_pos, i_neg, cols)
    plants the rows and columns of the overflow sums."""
    rng = np.random.default_rng(seed)
    r = rng.choice(row_scales, M)
    c = rng.choice(col_scales, N)
    A = rng.integers(0, r[:, None] + 1, (M, K))
    mixed = rng.random(M) < 0.125
    A[mixed] = rng.integers(-r[mixed, None], r[mixed, None] + 1, (int(mixed.sum()), K))
    A *= rng.choice([-1, 1], M)[:, None]
    B = rng.integers(0, c[None, :] + 1, (K, N))
    if plant is not None:
        i_pos, i_neg, cols = plant
        A[i_pos] = 16
        A[i_pos, K - 1] = 8
        if i_neg is not None:
            A[i_neg] = -A[i_pos]
        for j, (tot, last) in zip(cols, PLANTED):
            B[:, j] = column_with_sum(K, tot, last, fmt)
    if fmt == "e5m2":      # the few integers E5M2 lacks (9, 11, 13, 15) step down by one
        A = np.where(np.isin(np.abs(A), E5M2_INTS), A, A - np.sign(A))
        B = np.where(np.isin(B, E5M2_INTS), B, B - 1)
    return A, B


def rounding_census(S, fmt):
    """(outputs that need rounding, exact ties) among the exact sums S of a
    case, for a binary16 (f16, FP8 inputs) or bfloat16 output."""
    p = 11 if fmt != "bf16" else 8                 # significand bits
    a = np.abs(S).astype(np.int64)
    big = a >= (1 << p)
    e = np.floor(np.log2(np.maximum(a, 1))).astype(np.int64)
    ulp = np.left_shift(1, np.maximum(e - (p - 1), 0))
    rem = a % ulp
    return int(np.sum(big & (rem != 0))), int(np.sum(big & (2 * rem == ulp)))


def oracle_out(A, B, fmt, fa="e4m3", fb="e4m3"):
    """The oracle's output bits and exact sums for integer A [M, K], B [K, N]."""
    M, K = A.shape
    N = B.shape[1]
    if fmt in ("f16", "bf16"):
        Ab, Bb = to_format(A, fmt), to_format(B, fmt)
        return oracle.gemm(Ab, (K, 1), Bb, (N, 1), M, N, K, exact=True, dtype=fmt,
                           nthreads=ORACLE_THREADS)
    Ab, Bb = to_format(A, fa), to_format(B, fb)
    return oracle.gemm(Ab, (K, 1), Bb, (N, 1), M, N, K, exact=True, dtype="f8", fmt_a=fa, fmt_b=fb,
                       nthreads=ORACLE_THREADS)


def check_census(ref, S, fmt, plant, what, min_rounded=1000, min_ties=100):
    rounded, ties = rounding_census(S, fmt)
    assert rounded >= min_rounded and ties >= min_ties, f"{what}: {rounded} rounded, {ties} ties"
    if plant is not None and fmt != "bf16":
        i_pos, i_neg, cols = plant
        assert [int(x) for x in ref[i_pos, cols]] == PLANTED_BITS, what
        if i_neg is not None:
            assert [int(x) for x in ref[i_neg, cols]] == [b | 0x8000 for b in PLANTED_BITS], what


def dev16(vals, fmt, layout="row", pad=8):
    """Integer matrix -> device view of the 16-bit format, row-major or as a
    transposed view, rows padded with NaN."""
    bits = to_format(vals, fmt)
    R, C = bits.shape
    if layout == "col":
        bits = np.ascontiguousarray(bits.T)
        R, C = C, R
    buf = np.full((R, C + pad), NAN16 if fmt == "f16" else 0x7FC0, dtype=np.uint16)
    buf[:, :C] = bits
    t = torch.from_numpy(buf.view(np.int16)).to(DEV).view(TORCH_FMT[fmt])[:, :C]
    return t.t() if layout == "col" else t


def dev8(vals, fmt, layout="k"):
    """Integer matrix -> FP8 device view; "k": stored as given (rows padded
    to 16 bytes plus 16 with the NaN byte 0x7F); for B, "k" means the [N, K]
    storage (K-contiguous, passed as a transposed view), "n" the [K, N] one."""
    bits = to_format(vals, fmt)
    R, C = bits.shape
    if layout == "kT":                 # B given as [K, N] values, stored [N, K]
        bits = np.ascontiguousarray(bits.T)
        R, C = C, R
    pad = (-C) % 16 + 16
    buf = np.full((R, C + pad), 0x7F, dtype=np.uint8)
    buf[:, :C] = bits
    t = torch.from_numpy(buf).to(DEV).view(TORCH_FMT[fmt])[:, :C]
    return t.t() if layout == "kT" else t


def run(a, b, M, N, what, **kw):
    say(f"rounding {what} M={M} N={N} K={a.shape[1]} a.stride={a.stride()} b.stride={b.stride()} {kw}")
    out = Out(M, N, ldc=N + 4)
    view = out.view.view(torch.bfloat16) if a.dtype == torch.bfloat16 else out.view
    g.gemm(a, b, out=view, **kw)
    torch.cuda.synchronize()
    return out.result()


# ------------------------------------------------------------------ fp16, tile families

MAIN_PLANS = [
    ("dma256 tile 14", dict(variant="main", tile=14)),
    ("dma256 tile 13", dict(variant="main", tile=13)),
    ("dma128 tile 7", dict(variant="main", tile=7)),
    ("dma64x128 tile 8", dict(variant="main", tile=8)),
    ("register 256", dict(variant="main", tile=6)),
    ("register 128", dict(variant="main", tile=1)),
    ("64x32x32", dict(variant="tile64x32")),
    ("split-K 256 x3", dict(variant="splitk", tile=14, split_k=3)),
    ("split-K 128 x5", dict(variant="splitk", tile=1, split_k=5)),
    ("split-K dma128 x3", dict(variant="splitk", tile=7, split_k=3)),
    ("stream-K x3", dict(variant="streamk", split_k=3)),
    ("auto", dict(variant="auto")),
]


@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_fp16_rounding_tile_paths(b_layout):
    M, N, K = 600, 520, 384
    plant = (5, M - 3, [0, 131, 300, N - 1])
    A, B = int_inputs(M, N, K, 91001, plant=plant)
    ref, S = oracle_out(A, B, "f16")
    check_census(ref, S, "f16", plant, "fp16 tiles")
    a, b = dev16(A, "f16"), dev16(B, "f16", b_layout)
    for name, kw in MAIN_PLANS:
        p = g.plan(a, b, **kw)
        if "tile" in kw:
            assert p["tile_id"] == kw["tile"], (name, p)
        if kw["variant"] == "streamk":
            assert p["variant"] == "streamk" and p["sk_tiles"] > 0 and p["split_k"] == 3, p
        assert_bits_equal(run(a, b, M, N, name, **kw), ref, f"fp16 {name} B={b_layout} plan {p}")


def test_fp16_rounding_packed_b():
    M, N, K = 600, 520, 384
    plant = (7, 300, [1, 255, 256, N - 2])
    A, B = int_inputs(M, N, K, 91002, plant=plant)
    ref, S = oracle_out(A, B, "f16")
    check_census(ref, S, "f16", plant, "packed B")
    a = dev16(A, "f16")
    for layout in ("row", "col"):
        packed = g.pack_b(dev16(B, "f16", layout))
        out = Out(M, N, ldc=N + 4)
        say(f"rounding packed B={layout}")
        g.gemm_packed(a, packed, out=out.view)
        torch.cuda.synchronize()
        assert_bits_equal(out.result(), ref, f"packed B={layout}")


@pytest.mark.parametrize("M", [9, 20, 40, 64])
def test_fp16_rounding_skinny_tiles(M):
    N, K = 520, 1152
    plant = (0, M - 1, [3, 256, 257, N - 1])
    A, B = int_inputs(M, N, K, 91100 + M, row_scales=(2, 4, 8), plant=plant)
    ref, S = oracle_out(A, B, "f16")
    check_census(ref, S, "f16", plant, f"skinny M={M}", min_rounded=200, min_ties=20)
    a = dev16(A, "f16")
    for layout in ("row", "col"):
        b = dev16(B, "f16", layout)
        for kw in (dict(variant="skinny"), dict(variant="skinny", split_k=1),
                   dict(variant="skinny", split_k=5), dict(variant="auto")):
            p = g.plan(a, b, **kw)
            assert_bits_equal(run(a, b, M, N, f"skinny M={M}", **kw), ref,
                              f"skinny M={M} B={layout} plan {p}")


@pytest.mark.parametrize("b_layout", ["row", "col"])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_fp16_rounding_decode_kernel(M, b_layout):
    # Split counts 18, 5 and 3 reach the reduction with 16, 4 and 1 lanes per
    # output; split 1 stores from the decode kernel itself; 0 is automatic.
    # B N-contiguous, or as [N, K] rows (the kernel's K-contiguous form).
    N, K = 520, 1152
    plant = (0, M - 1 if M > 1 else None, [0, 255, 256, N - 1])
    A, B = int_inputs(M, N, K, 91200 + M, row_scales=(2, 4, 8), plant=plant)
    ref, S = oracle_out(A, B, "f16")
    check_census(ref, S, "f16", plant, f"decode M={M}", min_rounded=50, min_ties=5)
    a, b = dev16(A, "f16"), dev16(B, "f16", b_layout)
    for split in (0, 18, 5, 3, 1):
        p = g.plan(a, b, variant="skinny", split_k=split)
        assert p["tile_m"] == 16 and p["tile_n"] == 128, p
        assert p["b_path"] == ("kvec" if b_layout == "col" else "rvec"), p
        assert split == 0 or p["split_k"] == split, p
        assert_bits_equal(run(a, b, M, N, f"decode M={M}", variant="skinny", split_k=split), ref,
                          f"decode M={M} split {split} plan {p}")


def test_fp16_rounding_grouped():
    sizes = np.array([300, 0, 517, 40, 263])
    K, N = 384, 264
    offsets = np.concatenate([[2], 2 + np.cumsum(sizes)]).astype(np.int64)
    M = int(offsets[-1]) + 3
    G = len(sizes)
    A, _ = int_inputs(M, 1, K, 91300)
    Bs = np.stack([int_inputs(1, N, K, 91310 + e)[1] for e in range(G)])
    # plant the overflow sums in group 0 (its first two rows) and group 4
    for e, (ip, ineg) in ((0, (2, 3)), (4, (int(offsets[4]), int(offsets[5]) - 1))):
        A[ip] = 16
        A[ip, K - 1] = 8
        A[ineg] = -A[ip]
        for j, (tot, last) in zip([0, 100, 200, N - 1], PLANTED):
            Bs[e][:, j] = column_with_sum(K, tot, last, "f16")
    Ab = to_format(A, "f16")
    ref = np.full((M, N), NAN16, dtype=np.uint16)
    census = [0, 0]
    for e in range(G):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            ref[r0:r1], S = oracle.gemm(np.ascontiguousarray(Ab[r0:r1]), (K, 1),
                                        to_format(Bs[e], "f16"), (N, 1), r1 - r0, N, K, exact=True,
                                        nthreads=ORACLE_THREADS)
            census = [x + y for x, y in zip(census, rounding_census(S, "f16"))]
    assert census[0] >= 1000 and census[1] >= 100, census
    assert [int(x) for x in ref[2, [0, 100, 200, N - 1]]] == PLANTED_BITS
    for layout in ("row", "col"):
        b3 = torch.stack([dev16(Bs[e], "f16", layout) for e in range(G)]) if layout == "row" else \
            torch.from_numpy(to_format(np.ascontiguousarray(Bs.transpose(0, 2, 1)), "f16").view(
                np.int16)).to(DEV).view(torch.float16).transpose(1, 2)
        out = Out(M, N)
        say(f"rounding grouped B={layout}")
        g.gemm_grouped(dev16(A, "f16"), b3, torch.from_numpy(offsets).to(DEV), out=out.view)
        torch.cuda.synchronize()
        assert_bits_equal(out.result(), ref, f"grouped B={layout}")


# ------------------------------------------------------------------ bfloat16

@pytest.mark.parametrize("M,N,K,plans", [
    (600, 520, 384, [dict(variant="main", tile=14), dict(variant="main", tile=1),
                     dict(variant="main", tile=7), dict(variant="splitk", tile=7, split_k=3),
                     dict(variant="main", tile=8),
                     dict(variant="splitk", tile=14, split_k=3), dict(variant="splitk", split_k=5),
                     dict(variant="auto")]),
    (40, 520, 1152, [dict(variant="skinny"), dict(variant="skinny", split_k=5)]),
    (3, 520, 1152, [dict(variant="skinny"), dict(variant="skinny", split_k=5),
                    dict(variant="skinny", split_k=1)]),
])
def test_bf16_rounding(M, N, K, plans):
    A, B = int_inputs(M, N, K, 91400 + M, row_scales=(2, 4, 8))
    ref, S = oracle_out(A, B, "bf16")
    check_census(ref, S, "bf16", None, f"bf16 {M}x{N}x{K}", min_rounded=200, min_ties=20)
    a = dev16(A, "bf16")
    for layout in ("row", "col"):
        b = dev16(B, "bf16", layout)
        for kw in plans:
            p = g.plan(a, b, **kw)
            assert_bits_equal(run(a, b, M, N, f"bf16 {layout}", **kw), ref,
                              f"bf16 {M}x{N}x{K} B={layout} plan {p}")


# ------------------------------------------------------------------ FP8 operands, fp16 output

@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"),
                                   ("e5m2", "e5m2")])
def test_f8_rounding(fa, fb):
    M, N, K = 600, 528, 384
    plant = (5, M - 3, [0, 131, 300, N - 1])
    # B's values must suit fb, A's fa: draw each from the stricter set when
    # either is E5M2 (the planted sums use only 16, 8 and small integers).
    fmt = "e5m2" if "e5m2" in (fa, fb) else "e4m3"
    A, B = int_inputs(M, N, K, 91500, fmt=fmt, plant=plant)
    ref, S = oracle_out(A, B, "f8", fa, fb)
    check_census(ref, S, "f8", plant, f"f8 {fa}/{fb}")
    a = dev8(A, fa)
    for b_layout in ("kT", "n"):
        b = dev8(B, fb, b_layout)
        for kw in (dict(variant="main"), dict(variant="splitk", split_k=3),
                   dict(variant="streamk", split_k=3), dict(variant="auto")):
            p = g.plan(a, b, **kw)
            assert_bits_equal(run(a, b, M, N, f"f8 {fa}/{fb} B={b_layout}", **kw), ref,
                              f"f8 {fa}/{fb} B={b_layout} plan {p}")
    # grouped FP8: two groups over the same rows, B stacked twice
    offsets = np.array([0, 300, M], dtype=np.int64)
    b3 = torch.stack([dev8(B, fb, "kT"), dev8(B, fb, "kT")])
    out = Out(M, N)
    say(f"rounding f8 grouped {fa}/{fb}")
    g.gemm_grouped(a, b3, torch.from_numpy(offsets).to(DEV), out=out.view)
    torch.cuda.synchronize()
    assert_bits_equal(out.result(), ref, f"f8 grouped {fa}/{fb}")
