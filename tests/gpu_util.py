"""Helpers for the GPU parity tests: device transfer of fp16 bit arrays and
the acceptance checks against the oracle."""
import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"
ORACLE_THREADS = min(16, oracle.threads())


def say(*msg):
    """Name the case on stdout before each GPU step, so a crash is attributable."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    """numpy uint16 (fp16 bits) -> torch.float16 on the GPU, same shape."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.float16)


def to_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def val(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def tolerance_violations(gpu_bits, ref_bits):
    """Elementwise check of |C_gpu - C_oracle| <= 1e-2 + 2e-3 |C_oracle| with
    C_oracle the oracle's fp16 output; NaN anywhere is a violation.  Returns
    (number of violations, worst excess, index of the worst)."""
    g, r = val(gpu_bits), val(ref_bits)
    err = np.abs(g - r)
    bound = 1e-2 + 2e-3 * np.abs(r)
    bad = ~(err <= bound)                       # NaN counts as bad
    if not bad.any():
        return 0, 0.0, None
    excess = np.where(np.isnan(err), np.inf, err - bound)
    idx = np.unravel_index(np.argmax(excess), excess.shape)
    return int(bad.sum()), float(excess[idx]), idx


def assert_close(gpu_bits, ref_bits, what=""):
    n, worst, idx = tolerance_violations(gpu_bits, ref_bits)
    assert n == 0, (f"{what}: {n} outputs outside 1e-2 + 2e-3|C| (worst excess {worst} at {idx}: "
                    f"gpu {val(gpu_bits)[idx]} oracle {val(ref_bits)[idx]})")


def bf16_val(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def assert_close_bf16(gpu_bits, ref_bits, what=""):
    """bfloat16 outputs: |C_gpu - C_oracle| <= 1e-2 + 8e-3 |C_oracle| (one
    bfloat16 unit in the last place is at most 2^-7 |C|; the fp32 sums of the
    two sides may fall on either side of a rounding boundary)."""
    g, r = bf16_val(gpu_bits), bf16_val(ref_bits)
    err = np.abs(g - r)
    bad = ~(err <= 1e-2 + 8e-3 * np.abs(r))
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} bfloat16 outputs outside 1e-2 + 8e-3|C| "
                             f"(first at {idx}: gpu {g[idx]} oracle {r[idx]})")


def assert_bits_equal(gpu_bits, ref_bits, what=""):
    if not np.array_equal(gpu_bits, ref_bits):
        diff = np.argwhere(gpu_bits != ref_bits)
        i = tuple(diff[0])
        raise AssertionError(f"{what}: {len(diff)} outputs differ in bits; first at {i}: "
                             f"gpu {gpu_bits[i]:#06x} ({val(gpu_bits)[i]}) oracle "
                             f"{ref_bits[i]:#06x} ({val(ref_bits)[i]})")


def ulp_histogram(gpu_bits, ref_bits):
    """Distance in units in the last place between two fp16 arrays (finite)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    d = np.abs(ordered(gpu_bits) - ordered(ref_bits))
    return {int(k): int(v) for k, v in zip(*np.unique(d, return_counts=True))}


NAN16 = 0x7E00
CANARY = 0x5A5A


def dev_nan(n):
    return torch.full((n,), float("nan"), dtype=torch.float16, device=DEV)


def place(logical, layout, pad=(0, 0)):
    """Put a logical [R, C] fp16-bit matrix on the GPU and return a torch view
    of shape [R, C] with the requested storage:
      "row"  row-major, strides (C + pad[1], 1) inside a NaN buffer with
             pad[0] leading NaN rows (pad = (0, 0): a plain contiguous tensor)
      "col"  a transposed view: stored [C, R], strides (1, R + pad[1])."""
    R, Cc = logical.shape
    if layout == "row":
        if pad == (0, 0):
            return to_dev(logical)
        ld = Cc + pad[1]
        buf = dev_nan((R + pad[0] + 1) * ld)
        v = buf[pad[0] * ld: pad[0] * ld + R * ld].view(R, ld)[:, :Cc]
        v.copy_(to_dev(logical))
        return v
    if layout == "col":
        if pad == (0, 0):
            return to_dev(np.ascontiguousarray(logical.T)).t()
        ld = R + pad[1]
        buf = dev_nan((Cc + pad[0] + 1) * ld)
        v = buf[pad[0] * ld: pad[0] * ld + Cc * ld].view(Cc, ld)[:, :R]
        v.copy_(to_dev(np.ascontiguousarray(logical.T)))
        return v.t()
    raise ValueError(layout)


class Out:
    """An [M, N] output view with row stride ldc inside a buffer pre-filled
    with NaN (the view) and a canary pattern (everything else)."""

    def __init__(self, M, N, ldc=None, guard=64):
        ldc = ldc or N
        self.M, self.N, self.ldc, self.guard = M, N, ldc, guard
        host = np.full(guard + M * ldc + guard, CANARY, dtype=np.uint16)
        host[guard:guard + M * ldc].reshape(M, ldc)[:, :N] = NAN16
        self.buf = to_dev(host)
        self.view = self.buf[guard:guard + M * ldc].view(M, ldc)[:, :N]

    def result(self):
        host = to_host(self.buf)
        inner = host[self.guard:self.guard + self.M * self.ldc].reshape(self.M, self.ldc)
        assert np.all(host[:self.guard] == CANARY) and np.all(host[-self.guard:] == CANARY), \
            "write outside the output buffer"
        assert np.all(inner[:, self.N:] == CANARY), "write into the ldc padding"
        return np.ascontiguousarray(inner[:, :self.N])


def band_rows(M, tile=256):
    """One row per 256-row band of C, at an offset inside the band that
    varies from band to band, plus the first and last rows."""
    bands = np.arange((M + tile - 1) // tile, dtype=np.int64)
    rows = np.minimum(bands * tile + (bands * 37 + 11) % tile, M - 1)
    return np.unique(np.concatenate([rows, [0, M - 1]]))


def full_size_check(a, b, A, Bh, ldb, M, N, K, seed, what, points=100_000, dtype="f16",
                    fmt_a="e4m3", fmt_b="e4m3", band=256, **opts):
    """The automatic plan at full size, with every output checked for a
    writer and a sample checked against the oracle:
      - C starts as NaN and no element of the M x N output may still be NaN
        (counted on the device): every output has been written;
      - one oracle row per `band`-row band, at varying offsets in the band;
      - `points` outputs drawn uniformly over the whole of C, each computed
        by the oracle on its own.
    Both samples must meet 1e-2 + 2e-3 |C_oracle|; the distance in units in
    the last place is reported, and at least 95% of the points must agree
    bit for bit (an fp32 sum in another order rounds to the same fp16 value
    except near a rounding boundary).  Bh/ldb give the oracle B[k, j] =
    Bh.flat[k ldb[0] + j ldb[1]]; dtype "f8" takes FP8 bytes of formats
    fmt_a / fmt_b (fp16 output).  `opts` are passed to the call (the
    automatic plan by default)."""
    import dense_tiled_gemm_fp16_amd as g
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    p = g.plan(a, b, out=out, **opts)
    say(f"full size {what}: M={M} N={N} K={K} plan {p}")
    g.gemm(a, b, out=out, **opts)
    torch.cuda.synchronize()
    unwritten = int(torch.isnan(out).sum().item())
    assert unwritten == 0, f"{what}: {unwritten} outputs never written (still NaN)"
    rows = band_rows(M, band)
    gpu_rows = to_host(out[torch.from_numpy(rows).to(DEV)])
    ref_rows = oracle.gemm(np.ascontiguousarray(A[rows]), (K, 1), Bh, ldb, rows.size, N, K,
                           nthreads=ORACLE_THREADS, dtype=dtype, fmt_a=fmt_a, fmt_b=fmt_b)
    assert_close(gpu_rows, ref_rows, f"{what}: band rows")
    rng = np.random.default_rng(seed)
    pr = rng.integers(0, M, points)
    pc = rng.integers(0, N, points)
    gpu_pts = to_host(out[torch.from_numpy(pr).to(DEV), torch.from_numpy(pc).to(DEV)])
    ref_pts = oracle.gemm_points(A, (K, 1), Bh, ldb, K, pr, pc, nthreads=ORACLE_THREADS,
                                 dtype=dtype, fmt_a=fmt_a, fmt_b=fmt_b)
    assert_close(gpu_pts, ref_pts, f"{what}: random points")
    hist = ulp_histogram(gpu_pts, ref_pts)
    say(f"{what}: ulp distance of {points} points {hist}")
    assert hist.get(0, 0) >= 0.95 * points, f"{what}: ulp histogram {hist}"
    return p
