"""Seeded synthetic fp16 inputs, shared by the GPU tests, the CPU oracle and
the benchmark.

This package holds no matrix-multiply arithmetic: it only maps
(seed, tensor id, logical row, logical column) to a binary16 bit pattern with
a counter-based hash (SplitMix64, Steele, Lea and Flood, OOPSLA 2014), so any
element can be regenerated independently of how the matrix is stored.  A
matrix generated in row-major storage and the same matrix generated as a
transposed view hold identical logical values.

Modes:
  "uniform": U(-1, 1) drawn on the odd multiples of 2^-24, rounded to fp16
             with ties to even (the pages' workloads draw fp16 operands
             uniformly in [-1, 1]).
  "int":     integers in [-4, 4], exact in fp16 (for bit-exact checks).

`gen.c` is the fast path (threads over rows); `reference_rows` is a numpy
restatement of the same definition used to pin it.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
MODES = {"uniform": 0, "int": 1}
FORMATS = {"f16": 0, "bf16": 2, "e4m3": 4, "e5m2": 8}
F8 = ("e4m3", "e5m2")
TENSOR_A, TENSOR_B = 0, 1

_lib = None


def build():
    """Compile gen.c into libsynth.so next to it (gcc, no GPU involved)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
            ctypes.c_int]
        _lib = lib
    return _lib


def host_threads():
    """Worker threads: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def fill(dst, rows, cols, rs, cs, seed, tensor, mode="uniform", row0=0, row_index=None,
         nthreads=None, fmt="f16"):
    """Write logical element (row, c) of the (seed, tensor) matrix to
    dst.flat[r*rs + c*cs] for r in [0, rows).  The logical row is
    row_index[r] when row_index is given, else row0 + r.  `dst` is a
    uint16 numpy array (any shape, C-contiguous storage is addressed flat).
    fmt "f16" writes binary16 bits, "bf16" bfloat16 bits of the same value;
    "e4m3" / "e5m2" write OCP FP8 bytes into a uint8 array."""
    assert dst.dtype == (np.uint8 if fmt in F8 else np.uint16) and dst.flags["C_CONTIGUOUS"]
    if rows > 0 and cols > 0:
        last = (rows - 1) * rs + (cols - 1) * cs
        assert 0 <= last < dst.size, "fill would write outside dst"
    idx = None
    if row_index is not None:
        idx = np.ascontiguousarray(row_index, dtype=np.int64)
        assert idx.shape == (rows,)
    rc = _load().synth_fill(
        dst.ctypes.data, rows, cols, rs, cs, row0,
        None if idx is None else idx.ctypes.data,
        seed & 0xFFFFFFFFFFFFFFFF, tensor, MODES[mode] | FORMATS[fmt], nthreads or host_threads())
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return dst


def matrix(rows, cols, seed, tensor, mode="uniform", order="row", nthreads=None, fmt="f16"):
    """The logical [rows, cols] matrix as uint16 fp16 bits.

    order="row": returned array has shape (rows, cols) (row-major storage).
    order="col": returned array has shape (cols, rows) and holds the
    transpose, i.e. the storage of a transposed view with strides (1, rows)."""
    dt = np.uint8 if fmt in F8 else np.uint16
    if order == "row":
        out = np.empty((rows, cols), dtype=dt)
        return fill(out, rows, cols, cols, 1, seed, tensor, mode, nthreads=nthreads, fmt=fmt)
    if order == "col":
        out = np.empty((cols, rows), dtype=dt)
        return fill(out, rows, cols, 1, rows, seed, tensor, mode, nthreads=nthreads, fmt=fmt)
    raise ValueError(order)


def rows_of(row_index, cols, seed, tensor, mode="uniform", nthreads=None, fmt="f16"):
    """Selected logical rows (len(row_index), cols) of the (seed, tensor) matrix."""
    idx = np.ascontiguousarray(row_index, dtype=np.int64)
    out = np.empty((idx.size, cols), dtype=np.uint8 if fmt in F8 else np.uint16)
    return fill(out, idx.size, cols, cols, 1, seed, tensor, mode, row_index=idx,
                nthreads=nthreads, fmt=fmt)


def group_sizes(G, total, seed, skew=0.8):
    """Seeded row counts of G groups summing to `total` (e.g. tokens routed
    to each expert of a mixture-of-experts layer): weights (rank + 1)^-skew in
    a seeded random order, rounded down, the remainder given one row at a
    time to the heaviest groups.  Synthetic stand-in for routing data."""
    rng = np.random.default_rng(seed)
    w = (np.arange(G, dtype=np.float64) + 1.0) ** -skew
    w = w[rng.permutation(G)]
    sizes = np.floor(w / w.sum() * total).astype(np.int64)
    order = np.argsort(-w, kind="stable")
    for i in range(int(total - sizes.sum())):
        sizes[order[i % G]] += 1
    return sizes


# ---------------------------------------------------------------------------
# numpy restatement of the same definition (used only to pin gen.c)

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


def _sm(x):
    with np.errstate(over="ignore"):
        z = (x + np.uint64(0x9E3779B97F4A7C15)) & _M64
        z = ((z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)) & _M64
        z = ((z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)) & _M64
        return z ^ (z >> np.uint64(31))


def reference_rows(row_index, cols, seed, tensor, mode="uniform", fmt="f16"):
    rows = np.asarray(row_index, dtype=np.uint64).reshape(-1, 1)
    base_t = _sm(_sm(np.uint64(seed)) ^ np.uint64(tensor))
    h = _sm(_sm(base_t ^ rows) ^ np.arange(cols, dtype=np.uint64).reshape(1, -1))
    top = (h >> np.uint64(40)).astype(np.int64)
    if mode == "int":
        vals = (top % 9 - 4).astype(np.float32)
    else:
        vals = ((2 * top + 1 - (1 << 24)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
    if fmt == "bf16":   # float32 -> bfloat16, ties to even, by torch (values exact in float32)
        import torch
        return torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if fmt in F8:       # float32 -> OCP FP8, ties to even, by torch
        import torch
        dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
        return torch.from_numpy(vals).to(dt).view(torch.uint8).numpy()
    return vals.astype(np.float16).view(np.uint16)
