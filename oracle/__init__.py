"""CPU oracle for C = A.B with fp16 (or bfloat16) inputs and output, and
with FP8 (E4M3 / E5M2) inputs and fp16 output.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, the smoke check in
`__graft_entry__.py` and the CPU-baseline leg of `bench.py` may import this
package.  The GPU library (`dense_tiled_gemm_fp16_amd`) neither imports it
nor shares any code with it; the only thing the two sides have in common is
the seeded input generator in `synth/`, which holds no GEMM arithmetic.

Contents
  oracle.c  the defining triple loop in binary64 with a single
            round-to-nearest-even to binary16 (or bfloat16), and its own
            codecs for both formats (see that file's header for the passages
            it follows);
  model.py  a small pure-Python model of the tiled method (programs that own
            output tiles, K rounds, three-axis masks, read counting) used to
            reproduce the pages' worked examples;
  this file ctypes bindings with bounds checks on every buffer.

Parity status: the codec, the rounding, the masking, the stride and int64
examples, the read ledger and the tile geometry are pinned by the pages'
printed values, library routines and exact integer arithmetic (see
tests/test_oracle.py).  For non-integer U(-1,1) inputs the pages print no
output values, so those results rest on the definition plus the tolerance.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build():
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-shared", "-pthread", "-o", tmp, _SRC])
    os.replace(tmp, _LIB)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.orc_gemm_f16.restype = ctypes.c_int
        lib.orc_gemm_f16.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, i64, i64,
                                     ctypes.c_int]
        lib.orc_gemm_f16_points.restype = ctypes.c_int
        lib.orc_gemm_f16_points.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp, i64, vp,
                                            vp, ctypes.c_int]
        lib.orc_f16_to_f64_array.restype = None
        lib.orc_f16_to_f64_array.argtypes = [vp, vp, i64]
        lib.orc_f64_to_f16_array.restype = None
        lib.orc_f64_to_f16_array.argtypes = [vp, vp, i64]
        for name in ("orc_gemm_bf16",):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = lib.orc_gemm_f16.argtypes
        lib.orc_gemm_bf16_points.restype = ctypes.c_int
        lib.orc_gemm_bf16_points.argtypes = lib.orc_gemm_f16_points.argtypes
        lib.orc_bf16_to_f64_array.restype = None
        lib.orc_bf16_to_f64_array.argtypes = [vp, vp, i64]
        lib.orc_f64_to_bf16_array.restype = None
        lib.orc_f64_to_bf16_array.argtypes = [vp, vp, i64]
        lib.orc_gemm_f8.restype = ctypes.c_int
        lib.orc_gemm_f8.argtypes = lib.orc_gemm_f16.argtypes[:-1] + [ctypes.c_int] * 3
        lib.orc_gemm_f8_points.restype = ctypes.c_int
        lib.orc_gemm_f8_points.argtypes = lib.orc_gemm_f16_points.argtypes[:-1] + [ctypes.c_int] * 3
        for name in ("orc_e4m3_to_f64_array", "orc_e5m2_to_f64_array"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [vp, vp, i64]
        _lib = lib
    return _lib


def threads():
    """Worker threads: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def f16_to_f64(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().orc_f16_to_f64_array(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def f64_to_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_f16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_f64(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().orc_bf16_to_f64_array(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def f64_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


F8_FORMATS = {"e4m3": 0, "e5m2": 1}


def f8_to_f64(bits, fmt):
    """Decode FP8 bytes (uint8 array) of format "e4m3" (OCP E4M3FN) or "e5m2"."""
    wide = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.uint16)
    out = np.empty(wide.shape, dtype=np.float64)
    fn = {"e4m3": _load().orc_e4m3_to_f64_array, "e5m2": _load().orc_e5m2_to_f64_array}[fmt]
    fn(wide.ctypes.data, out.ctypes.data, wide.size)
    return out


def _widen_f8(buf, name):
    if not (isinstance(buf, np.ndarray) and buf.dtype == np.uint8 and buf.flags["C_CONTIGUOUS"]):
        raise TypeError(f"{name} must be a C-contiguous uint8 numpy array of FP8 bytes")
    return buf.astype(np.uint16)


def _span(off, rows, cols, rs, cs):
    """Largest element offset touched by a rows x cols view (strides >= 0)."""
    return off + (rows - 1) * rs + (cols - 1) * cs


def _check_buf(buf, name):
    if not (isinstance(buf, np.ndarray) and buf.dtype == np.uint16 and buf.flags["C_CONTIGUOUS"]):
        raise TypeError(f"{name} must be a C-contiguous uint16 numpy array of fp16 bits")


def gemm(A, lda, B, ldb, M, N, K, a_off=0, b_off=0, C=None, ldc=None, c_off=0,
         exact=False, nthreads=None, dtype="f16", fmt_a="e4m3", fmt_b="e4m3"):
    """C[i,j] = rne(sum_k A[i,k] B[k,j]) for the strided views
        A[i,k] = A.flat[a_off + i*lda[0] + k*lda[1]]
        B[k,j] = B.flat[b_off + k*ldb[0] + j*ldb[1]]
    written to C.flat[c_off + i*ldc + j] (a fresh (M, N) array when C is None).
    dtype "f16" (binary16) or "bf16" (bfloat16) for inputs and output, or
    "f8": A and B are uint8 FP8 bytes of formats fmt_a / fmt_b ("e4m3" or
    "e5m2") and C is binary16.
    Returns C, or (C, S) with S the unrounded binary64 sums when exact=True."""
    if dtype == "f8":
        A, B = _widen_f8(A, "A"), _widen_f8(B, "B")
    _check_buf(A, "A")
    _check_buf(B, "B")
    if min(M, N, K) <= 0:
        raise ValueError("empty shape is outside the contract")
    if min(lda + ldb) < 0:
        raise ValueError("negative stride")
    if _span(a_off, M, K, *lda) >= A.size or _span(b_off, K, N, *ldb) >= B.size:
        raise ValueError("view reaches past its buffer")
    if C is None:
        C = np.empty((M, N), dtype=np.uint16)
        ldc, c_off = N, 0
    _check_buf(C, "C")
    if ldc is None:
        ldc = N
    if _span(c_off, M, N, ldc, 1) >= C.size:
        raise ValueError("output view reaches past its buffer")
    S = np.empty((M, N), dtype=np.float64) if exact else None
    args = (A.ctypes.data + 2 * a_off, lda[0], lda[1], B.ctypes.data + 2 * b_off, ldb[0], ldb[1],
            C.ctypes.data + 2 * c_off, ldc, None if S is None else S.ctypes.data, M, N, K)
    if dtype == "f8":
        rc = _load().orc_gemm_f8(*args, F8_FORMATS[fmt_a], F8_FORMATS[fmt_b], nthreads or threads())
    else:
        fn = {"f16": _load().orc_gemm_f16, "bf16": _load().orc_gemm_bf16}[dtype]
        rc = fn(*args, nthreads or threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return (C, S) if exact else C


def gemm_grouped(A, Bs, offsets, N, K, C=None, nthreads=None, dtype="f16"):
    """Grouped product (TileLang tutorial ch. 14, section 4.3): for each group
    g, rows offsets[g] .. offsets[g+1]-1 of C are those rows of A times B_g,
    each by the plain definition of gemm() above.  A is [M, K] and Bs is
    [G, K, N] (row-major fp16 bits); rows of C outside every group keep their
    value (C is a fresh zero array when None)."""
    M = A.shape[0]
    G = Bs.shape[0]
    if len(offsets) != G + 1:
        raise ValueError("need G + 1 offsets")
    if C is None:
        C = np.zeros((M, N), dtype=np.uint16)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if not 0 <= r0 <= r1 <= M:
            raise ValueError("offsets must be non-decreasing inside [0, M]")
        if r1 > r0:
            C[r0:r1] = gemm(np.ascontiguousarray(A[r0:r1]), (K, 1), np.ascontiguousarray(Bs[g]),
                            (N, 1), r1 - r0, N, K, nthreads=nthreads, dtype=dtype)
    return C


def gemm_points(A, lda, B, ldb, K, rows, cols, a_off=0, b_off=0, exact=False, nthreads=None,
                dtype="f16", fmt_a="e4m3", fmt_b="e4m3"):
    """Selected outputs C[rows[t], cols[t]] of the same product, each computed
    on its own.  Returns output bits (and the unrounded sums when exact=True)."""
    if dtype == "f8":
        A, B = _widen_f8(A, "A"), _widen_f8(B, "B")
    _check_buf(A, "A")
    _check_buf(B, "B")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be equal-length vectors")
    if K <= 0:
        raise ValueError("empty K is outside the contract")
    if rows.size:
        if rows.min() < 0 or cols.min() < 0:
            raise ValueError("negative coordinate")
        if (a_off + int(rows.max()) * lda[0] + (K - 1) * lda[1] >= A.size
                or b_off + (K - 1) * ldb[0] + int(cols.max()) * ldb[1] >= B.size):
            raise ValueError("point reaches past its buffer")
    out = np.empty(rows.size, dtype=np.uint16)
    S = np.empty(rows.size, dtype=np.float64) if exact else None
    args = (A.ctypes.data + 2 * a_off, lda[0], lda[1], B.ctypes.data + 2 * b_off, ldb[0], ldb[1], K,
            rows.ctypes.data, cols.ctypes.data, rows.size, out.ctypes.data,
            None if S is None else S.ctypes.data)
    if dtype == "f8":
        rc = _load().orc_gemm_f8_points(*args, F8_FORMATS[fmt_a], F8_FORMATS[fmt_b],
                                        nthreads or threads())
    else:
        fn = {"f16": _load().orc_gemm_f16_points, "bf16": _load().orc_gemm_bf16_points}[dtype]
        rc = fn(*args, nthreads or threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return (out, S) if exact else out
